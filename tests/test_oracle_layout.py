"""Pins of the oracle's layout: a hand-worked example on the glossary's
8-experts-over-4-GPUs placement, a sequential first-come reference written as
plain loops, and the invariants of the pages (counts add up to T*k, every
(token, slot) pair lands exactly once, capacity drops are counted)."""

import json
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_packed_and_capacity():
    with open(os.path.join(GOLDEN, "layout_worked_example.json")) as f:
        ex = json.load(f)
    idx = np.array(ex["topk_idx"], dtype=np.int32)
    e, r = ex["num_experts"], ex["num_ranks"]
    assert [c // (e // r) for c in range(e)] == ex["expert_to_rank"]
    for mode, cap in (("packed", 0), ("capacity_1", 1)):
        got = O.layout(idx, e, r, cap)
        want = ex[mode]
        for name in ("expert_counts", "expert_offsets", "rank_counts",
                     "rank_offsets", "rank_token_counts", "dst_row", "src_pair"):
            assert got[name].tolist() == want[name], (mode, name)
        assert int(got["overflow"][0]) == want["overflow"]


def _sequential_layout(idx, e, r, cap):
    """First-come reference: walk the pairs in row-major order with one
    running counter per expert (pure Python, small inputs only)."""
    t, k = idx.shape
    counts = [0] * e
    for row in idx:
        for v in row:
            if v >= 0:
                counts[v] += 1
    if cap == 0:
        starts = [0] * (e + 1)
        for c in range(e):
            starts[c + 1] = starts[c] + counts[c]
    else:
        starts = [c * cap for c in range(e + 1)]
    seen = [0] * e
    dst = [[-1] * k for _ in range(t)]
    for i in range(t):
        for j in range(k):
            v = int(idx[i, j])
            if v < 0:
                continue
            p = seen[v]
            seen[v] += 1
            if cap == 0 or p < cap:
                dst[i][j] = starts[v] + p
    return counts, starts, dst


CASES = [
    # tokens, experts, top_k, ranks, capacity, distinct, mask_frac
    (37, 8, 2, 4, 0, True, 0.0),
    (200, 16, 4, 4, 0, False, 0.0),      # duplicate experts inside a token
    (200, 16, 4, 8, 0, True, 0.2),       # masked slots
    (300, 8, 3, 2, 20, False, 0.1),      # capacity with drops
    (64, 32, 8, 32, 5, True, 0.0),
    (1, 4, 4, 1, 0, True, 0.0),
    (50, 6, 1, 3, 0, True, 0.5),
]


@pytest.mark.parametrize("case", CASES)
def test_layout_matches_sequential_reference(case):
    t, e, k, r, cap, distinct, mf = case
    g = np.random.Generator(np.random.PCG64(sum(case[:5])))
    idx = W.random_topk_idx(g, t, e, k, distinct=distinct, mask_frac=mf)
    got = O.layout(idx, e, r, cap)
    counts, starts, dst = _sequential_layout(idx, e, r, cap)
    assert got["expert_counts"].tolist() == counts
    assert got["expert_offsets"].tolist() == starts
    assert got["dst_row"].tolist() == dst


@pytest.mark.parametrize("case", CASES)
def test_layout_invariants(case):
    t, e, k, r, cap, distinct, mf = case
    g = np.random.Generator(np.random.PCG64(1000 + sum(case[:5])))
    idx = W.random_topk_idx(g, t, e, k, distinct=distinct, mask_frac=mf)
    L = O.layout(idx, e, r, cap)
    live = idx >= 0
    n_live = int(live.sum())
    cnt, off, dst, src = (L["expert_counts"], L["expert_offsets"],
                          L["dst_row"], L["src_pair"])
    epr = e // r
    assert cnt.sum() == n_live                          # counts add up
    assert np.all(dst[~live] == -1)
    kept = dst[live]
    kept = kept[kept >= 0]
    assert len(np.unique(kept)) == len(kept)             # each row used once
    if cap == 0:
        assert L["num_rows"] == t * k
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
        assert np.array_equal(np.sort(kept), np.arange(n_live))  # bijection
        assert L["overflow"][0] == 0
    else:
        assert L["num_rows"] == e * cap
        assert np.array_equal(off, np.arange(e + 1) * cap)
        assert np.minimum(cnt, cap).sum() + L["overflow"][0] == n_live
    # src_pair is the inverse of dst_row
    flat = dst.reshape(-1)
    for p in np.nonzero(flat >= 0)[0]:
        assert src[flat[p]] == p
    assert (src >= 0).sum() == (flat >= 0).sum()
    # stability: inside each expert's region the pairs stay in row-major order
    for c in range(e):
        seg = src[off[c]: off[c + 1]]
        seg = seg[seg >= 0]
        assert np.all(np.diff(seg) > 0)
        assert np.all(idx.reshape(-1)[seg] == c)
    # rank regions are whole experts (glossary placement rule)
    assert np.array_equal(L["rank_offsets"], off[::epr])
    rows_per_expert = np.minimum(cnt, cap) if cap else cnt
    assert np.array_equal(L["rank_counts"], rows_per_expert.reshape(r, epr).sum(axis=1))
    # distinct tokens per rank, counted the slow way
    rtc = [len({i for i in range(t) for j in range(k)
                if idx[i, j] >= 0 and idx[i, j] // epr == q}) for q in range(r)]
    assert L["rank_token_counts"].tolist() == rtc


def test_all_tokens_on_one_expert():
    t, e, k = 100, 8, 1
    idx = np.full((t, k), 5, dtype=np.int32)
    L = O.layout(idx, e, 4, 0)
    assert L["expert_counts"].tolist() == [0, 0, 0, 0, 0, 100, 0, 0]
    assert L["dst_row"][:, 0].tolist() == list(range(100))
    L = O.layout(idx, e, 4, 30)
    assert L["overflow"][0] == 70
    assert L["dst_row"][:30, 0].tolist() == list(range(150, 180))
    assert np.all(L["dst_row"][30:] == -1)


def test_all_masked():
    idx = np.full((10, 2), -1, dtype=np.int32)
    L = O.layout(idx, 4, 2, 0)
    assert L["expert_counts"].sum() == 0
    assert np.all(L["src_pair"] == -1) and np.all(L["dst_row"] == -1)
