"""Pins of the oracle's routing: brute-force top-k and group-limited top-k on
small inputs, closed forms of the weights, and the invariants the pages fix
(k distinct experts per token; destinations limited to the kept groups)."""

import itertools
import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W


def _beats(ka, ea, kb, eb):
    """Expert a comes before expert b in the top-k order (key desc, index asc)."""
    return ka > kb or (ka == kb and ea < eb)


def _brute_topk(key_row, allowed, k):
    """Slot j holds the allowed expert beaten by exactly j allowed experts."""
    cand = [e for e in range(len(key_row)) if allowed[e]]
    out = []
    for e in cand:
        rank = sum(1 for f in cand if f != e and _beats(key_row[f], f, key_row[e], e))
        if rank < k:
            out.append((rank, e))
    out.sort()
    assert [r for r, _ in out] == list(range(k))
    return [e for _, e in out]


@pytest.mark.parametrize("seed", range(5))
def test_softmax_topk_brute_force_with_ties(seed):
    g = np.random.Generator(np.random.PCG64(seed))
    t, e, k = 64, 12, 3
    # small integers force many exact ties between experts
    logits = g.integers(-3, 4, size=(t, e)).astype(np.float32)
    bias = (g.integers(-2, 3, size=e) * 0.5).astype(np.float32) if seed % 2 else None
    idx, w = O.route_softmax_topk(logits, k, bias)
    key = logits + (bias if bias is not None else 0)
    for i in range(t):
        assert idx[i].tolist() == _brute_topk(key[i], [True] * e, k)
        # weights: softmax of the raw logits over the chosen experts (fsum)
        ex = [math.exp(float(logits[i, c])) for c in idx[i]]
        s = math.fsum(ex)
        for j in range(k):
            want = np.float32(ex[j] / s)
            assert abs(w[i, j] - want) <= np.spacing(want)


def test_softmax_k2_weight_is_logistic_of_gap():
    g = np.random.Generator(np.random.PCG64(3))
    logits = g.standard_normal((1000, 8), dtype=np.float32)
    idx, w = O.route_softmax_topk(logits, 2)
    l0 = logits[np.arange(1000), idx[:, 0]].astype(np.float64)
    l1 = logits[np.arange(1000), idx[:, 1]].astype(np.float64)
    w0 = 1.0 / (1.0 + np.exp(l1 - l0))       # closed form for two experts
    assert np.all(np.abs(w[:, 0] - w0) <= np.spacing(w0.astype(np.float32)))
    assert np.all(w[:, 0] >= w[:, 1])       # the larger logit gets more weight


def test_sigmoid_scores_and_group_score_forms():
    g = np.random.Generator(np.random.PCG64(5))
    logits = g.standard_normal((50, 16), dtype=np.float32)
    s = O._sigmoid_f32(logits)
    ref = np.array([[np.float32(1.0 / (1.0 + math.exp(-float(v)))) for v in r]
                    for r in logits])
    assert np.array_equal(s, ref)
    key = s + np.float32(0.25)
    gs = O.group_scores(key.astype(np.float32), 4)
    for i in range(50):
        for gi in range(4):
            grp = key[i, 4 * gi: 4 * gi + 4]
            best = max(np.float32(grp[a] + grp[b])
                       for a, b in itertools.combinations(range(4), 2))
            assert gs[i, gi] == best            # largest pair sum = top-2 sum


@pytest.mark.parametrize("seed", range(4))
def test_group_limited_brute_force(seed):
    """E=16 in G=4 groups, keep 2 groups, pick 4: enumerate all group subsets;
    the kept subset is the one whose every member beats every non-member."""
    g = np.random.Generator(np.random.PCG64(100 + seed))
    t, e, G, kg, k = 80, 16, 4, 2, 4
    logits = (g.integers(-4, 5, size=(t, e)) * 0.5).astype(np.float32)
    bias = (g.integers(-1, 2, size=e) * 0.125).astype(np.float32)
    idx, w = O.route_group_limited(logits, k, G, kg, bias)
    s = np.array([[np.float32(1.0 / (1.0 + math.exp(-float(v)))) for v in r]
                  for r in logits], dtype=np.float32)
    key = (s + bias).astype(np.float32)
    gsz = e // G
    for i in range(t):
        score = [max(np.float32(key[i, gsz * q + a] + key[i, gsz * q + b])
                     for a, b in itertools.combinations(range(gsz), 2))
                 for q in range(G)]
        chosen = None
        for sub in itertools.combinations(range(G), kg):
            rest = [q for q in range(G) if q not in sub]
            if all(_beats(score[a], a, score[b], b) for a in sub for b in rest):
                assert chosen is None
                chosen = set(sub)
        allowed = [(c // gsz) in chosen for c in range(e)]
        assert idx[i].tolist() == _brute_topk(key[i], allowed, k)
        ss = [float(s[i, c]) for c in idx[i]]
        tot = math.fsum(ss)
        for j in range(k):
            want = np.float32(ss[j] / tot)
            assert abs(w[i, j] - want) <= np.spacing(want)


def test_dsv3_invariants():
    w = W.WORKLOADS["dsv3"]
    inp = W.make_inputs(w, 0, tokens=1024)
    idx, wt = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    gsz = w.experts // w.groups
    for r in idx:
        assert len(set(r.tolist())) == w.top_k
        assert len(set((r // gsz).tolist())) <= w.topk_groups
        # each group spans 4 of the 32 ranks, so at most 16 ranks per token
        assert len(set((r // w.experts_per_rank).tolist())) <= 16
    assert np.all(wt > 0)
    s = wt.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= w.top_k * 2.0 ** -24)
    # slot order is descending selection key
    sig = O._sigmoid_f32(inp.logits)
    key = (sig + inp.bias).astype(np.float32)
    ks = np.take_along_axis(key, idx, axis=1)
    assert np.all(np.diff(ks, axis=1) <= 0)


def test_sigmoid_without_groups_or_bias_equals_logit_topk():
    g = np.random.Generator(np.random.PCG64(9))
    # logits spaced well apart so fp32 sigmoid keeps them distinct
    logits = np.stack([g.permutation(32) * 0.1 for _ in range(40)]).astype(np.float32)
    idx, _ = O.route_group_limited(logits, 5, 1, 1, None)
    want = np.argsort(-logits, axis=1, kind="stable")[:, :5]
    assert np.array_equal(idx, want)


def test_qwen3_skew_load_is_about_ten_times_mean():
    w = W.WORKLOADS["qwen3_skew"]
    inp = W.make_inputs(w, 0)
    idx, _ = O.route(inp.logits, w.top_k, w.score_fn, bias=inp.bias)
    c = np.bincount(idx.ravel(), minlength=w.experts)
    ratio = c.max() / (w.tokens * w.top_k / w.experts)
    assert 9.5 <= ratio <= 10.5


@pytest.mark.parametrize("t,e,k,fn,G,kg", [(5, 256, 8, 1, 8, 4), (3, 512, 32, 1, 16, 8),
                                           (4, 256, 8, 0, 1, 1), (6, 128, 8, 1, 4, 2)])
def test_all_keys_equal_picks_the_lowest_experts(t, e, k, fn, G, kg):
    """Every key equal: all group scores tie, so groups 0..kg-1 are kept (ties to the lower
    group), and inside them every key ties, so experts 0..k-1 are chosen in index order (ties
    to the lower expert). Each weight is s / (k*s) or exp(0) / k, i.e. 1/k to rounding."""
    logits = np.full((t, e), 0.25, dtype=np.float32)
    idx, w = O.route(logits, k, fn, G, kg, None)
    assert (idx == np.arange(k)[None, :]).all()
    assert np.abs(w.astype(np.float64) - 1.0 / k).max() <= 2.0 ** -23
