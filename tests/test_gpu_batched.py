"""GPU parity of the batched entry points: moe_route_batched,
moe_layout_batched and moe_rank_layout_batched give, for every batch, the
bits that moe_route, moe_layout and moe_rank_layout give on that batch alone
(and hence the oracle's, which the single-call parity tests pin). Outputs
are poisoned with a value the calls never write, and followed by guard
entries."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import combine_moe_layout_06_amd as M  # noqa: E402
from gpu_helpers import dev, host  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402

GUARD = 8
POISON = 0x7B7B7B7B


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


def _ints(n):
    return torch.full((n + GUARD,), POISON, dtype=torch.int32, device="cuda")


ROUTE_CASES = [
    # batches, T, E, k, score, G, kg, bias
    (4, 4096, 256, 8, 1, 8, 4, True),     # DeepSeek-V3 routing shape
    (8, 128, 256, 8, 1, 8, 4, True),      # decode steps
    (3, 1000, 8, 2, 0, 1, 1, False),      # 8-lane teams
    (2, 333, 128, 8, 1, 4, 2, True),      # 16-lane teams with groups
    (5, 77, 512, 32, 1, 16, 8, True),     # one wave per token, k = 32
    (1, 300, 96, 4, 1, 1, 1, True),       # one batch
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: "nb%d_T%d_E%d_k%d" % c[:4])
def test_route_batched_equals_single_calls(case):
    nb, t, e, k, fn, G, kg, with_bias = case
    say("batched route", case)
    g = W.rng(sum(case[:4]) + 3)
    logits = [dev(g.standard_normal((t, e), dtype=np.float32)) for _ in range(nb)]
    # each batch its own bias (the last batch none)
    bias = [dev((g.standard_normal(e, dtype=np.float32) * np.float32(0.1)).astype(np.float32))
            if with_bias and b < nb - 1 else None for b in range(nb)]
    got = [(_ints(t * k), torch.full((t * k + GUARD,), float("nan"), device="cuda"))
           for _ in range(nb)]
    M.moe_route_batched(t, e, k, [(logits[b], bias[b], got[b][0], got[b][1]) for b in range(nb)],
                        fn, G, kg)
    for b in range(nb):
        idx = _ints(t * k)
        w = torch.full((t * k + GUARD,), float("nan"), device="cuda")
        M.moe_route(t, e, k, logits[b], bias[b], fn, G, kg, idx, w)
        assert torch.equal(got[b][0], idx), (case, b, "topk_idx")
        assert torch.equal(got[b][1][:t * k], w[:t * k]), (case, b, "topk_weights")
        assert torch.isnan(got[b][1][t * k:]).all(), (case, b, "write past topk_weights")
        assert (host(got[b][0])[t * k:] == POISON).all(), (case, b, "write past topk_idx")


class LayoutOut:
    def __init__(self, t, e, k, r, cap, rtc):
        rows = e * cap if cap else t * k
        self.n = dict(expert_counts=e, expert_offsets=e + 1, rank_counts=r, rank_offsets=r + 1,
                      dst_row=t * k, src_pair=rows, overflow=1)
        if rtc:
            self.n["rank_token_counts"] = r
        self.bufs = {name: _ints(max(n, 1)) for name, n in self.n.items()}
        self.wsb = M.moe_layout_workspace_bytes(t, e, k)
        self.ws = torch.empty(max(self.wsb, 4), dtype=torch.uint8, device="cuda")

    def io(self, idx):
        d = dict(self.bufs, topk_idx=idx, workspace=self.ws, workspace_bytes=self.wsb)
        d.setdefault("rank_token_counts", None)
        return d

    def result(self):
        out = {}
        for name, n in self.n.items():
            a = host(self.bufs[name])
            assert (a[max(n, 1):] == POISON).all(), ("write past", name)
            out[name] = a[:n]
        return out


LAYOUT_CASES = [
    # batches, T, E, k, R, cap, rank token counts, mask fraction
    (4, 4096, 256, 8, 32, 0, True, 0.0),      # DeepSeek-V3 layout: count + place
    (8, 128, 256, 8, 32, 128, True, 0.0),     # decode steps: one tile each
    (3, 16384, 8, 2, 8, 0, True, 0.0),        # mixtral shape
    (2, 8192, 128, 8, 16, 0, False, 0.05),    # qwen3 shape, masked slots
    (5, 513, 64, 2, 64, 7, True, 0.3),        # capacity with drops, two tiles
    (2, 70000, 64, 4, 8, 4300, True, 0.1),    # scan pass: batches one after the other
    (1, 100, 6, 4, 3, 0, True, 0.1),          # one batch, one tile
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=lambda c: "nb%d_T%d_E%d_k%d_R%d_cap%d" % c[:6])
def test_layout_batched_equals_single_calls(case):
    nb, t, e, k, r, cap, rtc, mf = case
    say("batched layout", case)
    g = W.rng(sum(case[:6]) + 5)
    idx_h = [W.random_topk_idx(g, t, e, k, distinct=True, mask_frac=mf) for _ in range(nb)]
    idx = [dev(a) for a in idx_h]
    outs = [LayoutOut(t, e, k, r, cap, rtc) for _ in range(nb)]
    M.moe_layout_batched(t, e, k, r, cap, [outs[b].io(idx[b]) for b in range(nb)])
    for b in range(nb):
        got = outs[b].result()
        one = LayoutOut(t, e, k, r, cap, rtc)
        o = one.io(idx[b])
        M.moe_layout(t, e, k, r, cap, idx[b], o["expert_counts"], o["expert_offsets"],
                     o["rank_counts"], o["rank_offsets"], o["rank_token_counts"], o["dst_row"],
                     o["src_pair"], o["overflow"], o["workspace"], o["workspace_bytes"])
        want = one.result()
        for name in want:
            assert np.array_equal(got[name], want[name]), (case, b, name)
    # and the oracle, on the first and last batch (small enough cases)
    if t * k <= 40000:
        for b in (0, nb - 1):
            L = O.layout(idx_h[b], e, r, cap)
            got = outs[b].result()
            for name in got:
                assert np.array_equal(got[name], L[name].reshape(got[name].shape)), (case, b, name)


class RankOut:
    def __init__(self, t, e, k, r):
        self.n = dict(rank_token_counts=r, rank_token_offsets=r + 1, rank_row=t * k,
                      send_row=t * k, row_token=t * min(k, r))
        self.bufs = {name: _ints(max(n, 1)) for name, n in self.n.items()}
        self.wsb = M.moe_rank_layout_workspace_bytes(t, k, r)
        self.ws = torch.empty(max(self.wsb, 4), dtype=torch.uint8, device="cuda")

    def io(self, idx):
        return dict(self.bufs, topk_idx=idx, workspace=self.ws, workspace_bytes=self.wsb)

    def single(self, t, e, k, r, idx):
        b = self.bufs
        M.moe_rank_layout(t, e, k, r, idx, b["rank_token_counts"], b["rank_token_offsets"],
                          b["rank_row"], b["send_row"], b["row_token"], self.ws, self.wsb)

    def result(self):
        out = {}
        for name, n in self.n.items():
            a = host(self.bufs[name])
            assert (a[max(n, 1):] == POISON).all(), ("write past", name)
            out[name] = a[:n]
        return out


RANK_CASES = [
    # batches, T, E, k, R, mask fraction
    (8, 4096, 256, 8, 8, 0.0),        # DeepSeek-V3 (token, rank) layout: count + place
    (8, 128, 256, 8, 8, 0.0),         # decode steps: one tile each
    (3, 16384, 8, 2, 8, 0.05),        # mixtral shape, masked slots
    (2, 8192, 128, 8, 16, 0.1),       # qwen3 shape
    (2, 70000, 64, 4, 64, 0.1),       # scan pass: one scan launch per batch
    (1, 100, 6, 4, 3, 0.2),           # one batch, one tile
    (3, 0, 8, 2, 4, 0.0),             # no tokens
    (3, 300, 512, 32, 512, 0.05),     # maximum sizes: one expert per rank, k = 32
    (8, 2000, 512, 32, 16, 0.0),      # k = 32, 63 tiles, every batch slot used
    (4, 1001, 12, 3, 3, 0.1),         # R not a power of two, ragged last tile
]


@pytest.mark.parametrize("case", RANK_CASES, ids=lambda c: "nb%d_T%d_E%d_k%d_R%d" % c[:5])
def test_rank_layout_batched_equals_single_calls(case):
    nb, t, e, k, r, mf = case
    say("batched rank layout", case)
    g = W.rng(sum(case[:5]) + 11)
    idx_h = [W.random_topk_idx(g, t, e, k, distinct=True, mask_frac=mf) for _ in range(nb)]
    idx = [dev(a) if t > 0 else torch.empty(0, dtype=torch.int32, device="cuda")
           for a in idx_h]
    outs = [RankOut(t, e, k, r) for _ in range(nb)]
    M.moe_rank_layout_batched(t, e, k, r, [outs[b].io(idx[b]) for b in range(nb)])
    for b in range(nb):
        got = outs[b].result()
        one = RankOut(t, e, k, r)
        one.single(t, e, k, r, idx[b])
        want = one.result()
        for name in want:
            assert np.array_equal(got[name], want[name]), (case, b, name)
    if 0 < t * k <= 40000:                     # and the oracle, on the first and last batch
        for b in (0, nb - 1):
            L = O.rank_layout(idx_h[b], e, r)
            got = outs[b].result()
            for name in got:
                assert np.array_equal(got[name], L[name].reshape(got[name].shape)), (case, b, name)


N_RANDOM = 40


def _draw(seed):
    g = W.rng(70000 + seed)
    nb = int(g.integers(1, M.MOE_MAX_BATCHES + 1))
    R = int(g.choice([1, 2, 4, 8, 16, 32]))
    E = R * int(g.choice([1, 2, 4, 8]))
    k = int(g.integers(1, min(E, 16) + 1))
    T = int(g.choice([1, 63, 64, 65, 127, 128, 129, int(g.integers(1, max(2, 20000 // k)))]))
    cap = 0 if g.random() < 0.5 else int(g.integers(1, max(2, 2 * T * k // E + 2)))
    # routing settings: softmax, or group-limited sigmoid when the experts split into groups
    G = int(g.choice([d for d in (1, 2, 4, 8) if E % d == 0 and E // d * d == E]))
    fn = 1 if G > 1 or g.random() < 0.5 else 0
    kg = int(g.integers(1, G + 1))
    while kg * (E // G) < k:
        kg += 1
    return dict(nb=nb, T=T, E=E, k=k, R=R, cap=cap, G=G, fn=fn, kg=kg,
                rtc=bool(g.random() < 0.7), seed=seed)


@pytest.mark.parametrize("seed", range(N_RANDOM))
def test_batched_random_shapes(seed):
    """Seeded random shapes through the three batched calls, each batch
    against the single calls on the same inputs, bit for bit."""
    c = _draw(seed)
    say("batched random case", c)
    nb, t, e, k, r, cap = c["nb"], c["T"], c["E"], c["k"], c["R"], c["cap"]
    g = W.rng(80000 + seed)
    logits = [dev(g.standard_normal((t, e), dtype=np.float32)) for _ in range(nb)]
    bias = [dev((g.standard_normal(e, dtype=np.float32) * np.float32(0.1)).astype(np.float32))
            if g.random() < 0.5 else None for _ in range(nb)]
    idx = [_ints(t * k) for _ in range(nb)]
    wts = [torch.full((t * k + GUARD,), float("nan"), device="cuda") for _ in range(nb)]
    M.moe_route_batched(t, e, k, [(logits[b], bias[b], idx[b], wts[b]) for b in range(nb)],
                        c["fn"], c["G"], c["kg"])
    outs = [LayoutOut(t, e, k, r, cap, c["rtc"]) for _ in range(nb)]
    M.moe_layout_batched(t, e, k, r, cap, [outs[b].io(idx[b]) for b in range(nb)])
    for b in range(nb):
        i1 = _ints(t * k)
        w1 = torch.full((t * k + GUARD,), float("nan"), device="cuda")
        M.moe_route(t, e, k, logits[b], bias[b], c["fn"], c["G"], c["kg"], i1, w1)
        assert torch.equal(idx[b], i1), (c, b, "topk_idx")
        assert torch.equal(wts[b][:t * k], w1[:t * k]), (c, b, "topk_weights")
        got = outs[b].result()
        one = LayoutOut(t, e, k, r, cap, c["rtc"])
        o = one.io(i1)
        M.moe_layout(t, e, k, r, cap, i1, o["expert_counts"], o["expert_offsets"],
                     o["rank_counts"], o["rank_offsets"], o["rank_token_counts"], o["dst_row"],
                     o["src_pair"], o["overflow"], o["workspace"], o["workspace_bytes"])
        want = one.result()
        for name in want:
            assert np.array_equal(got[name], want[name]), (c, b, name)
    rk = [RankOut(t, e, k, r) for _ in range(nb)]
    M.moe_rank_layout_batched(t, e, k, r, [rk[b].io(idx[b]) for b in range(nb)])
    for b in range(nb):
        one = RankOut(t, e, k, r)
        one.single(t, e, k, r, idx[b])
        got, want = rk[b].result(), one.result()
        for name in want:
            assert np.array_equal(got[name], want[name]), (c, b, "rank", name)
