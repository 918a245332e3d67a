"""The benchmark's pipelined steps (the route and layout of a group of steps
on a side stream beside the dispatch and combine of the group before, 2 *
group layer buffers in turn) give the same results as the same steps run one
after the other: eager, and captured in a HIP graph and replayed."""

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import combine_moe_layout_06_amd as M  # noqa: E402
from gpu_helpers import dev  # noqa: E402
from synth import workloads as W  # noqa: E402

NAMES = ("topk_idx", "topk_weights", "dst_row", "src_pair", "expert_counts", "expert_offsets",
         "rank_counts", "rank_token_counts", "overflow", "combined")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    M.lib()
    yield
    torch.cuda.synchronize()


def _state(b):
    out = {n: getattr(b, n).clone() for n in NAMES}
    live = b.src_pair >= 0
    out["rows"] = b.dispatched[live].clone()
    if b.scales is not None:
        out["scales"] = b.scales[live].clone()
    return out


def _poison(bufs):
    for b in bufs:
        for n in NAMES:
            v = getattr(b, n)
            v.fill_(-7.0 if v.dtype == torch.float32 else -7)
        b.dispatched.fill_(0x55)


@pytest.mark.parametrize("name,steps,group", [("dsv3", 10, 4), ("dsv3", 5, 1), ("decode", 11, 4)])
def test_pipelined_steps_equal_serial_steps(name, steps, group):
    w = W.WORKLOADS[name]
    say("pipelined steps", name, "x", steps, "in groups of", group)
    seeds = [w.step_seed0 + i for i in range(steps)] if w.steps > 1 else [0]
    inputs = []
    for s in seeds:
        inp = W.make_inputs(w, s)
        inputs.append(dict(logits=dev(inp.logits),
                           bias=dev(inp.bias) if inp.bias is not None else None,
                           x=dev(inp.x)))
    bufs = [M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                    dtype=w.dispatch_dtype) for _ in range(2 * group)]
    g = np.random.Generator(np.random.PCG64(3))
    y = dev(W.random_bf16_rows(g, bufs[0].num_rows, w.hidden))

    # serial reference of the last two steps, each alone in bufs[0]
    want = {}
    for i in (steps - 2, steps - 1):
        bench.serial_steps(w, bufs, inputs, y, i, 1)
        torch.cuda.synchronize()
        want[i] = _state(bufs[0])

    side = torch.cuda.Stream()
    _poison(bufs)
    bench.overlapped_steps(torch, w, bufs, inputs, y, 0, steps, side, group)
    torch.cuda.synchronize()
    for i in (steps - 2, steps - 1):
        got = _state(bufs[i % (2 * group)])
        for n, v in want[i].items():
            assert torch.equal(got[n], v), ("eager", i, n)
    say("  eager pipelined steps equal the serial ones")

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        bench.overlapped_steps(torch, w, bufs, inputs, y, 0, steps, side, group)
    for rep in range(2):
        _poison(bufs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in (steps - 2, steps - 1):
            got = _state(bufs[i % (2 * group)])
            for n, v in want[i].items():
                assert torch.equal(got[n], v), ("graph", rep, i, n)
    say("  graph replays equal the serial steps")


def test_pipelined_hierarchical_steps_equal_serial_steps():
    """The hierarchical pass pipelined the same way (route, expert layout and
    (token, rank) layout of a group beside the send, fan-out and combines of
    the group before), replayed from a graph, against the same steps run one
    after the other."""
    w = W.WORKLOADS["dsv3"]
    group, steps = 2, 6
    inp = W.make_inputs(w, 0)
    inputs = [dict(logits=dev(inp.logits), bias=dev(inp.bias), x=dev(inp.x))]
    sets = [(M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, 0,
                                     dtype=w.dispatch_dtype),
             M.RankBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks,
                                    dtype=w.dispatch_dtype))
            for _ in range(2 * group)]
    g = np.random.Generator(np.random.PCG64(4))
    y = dev(W.random_bf16_rows(g, sets[0][0].num_rows, w.hidden))
    bench.hierarchical_front(w, sets, inputs, 0, 0)
    bench.hierarchical_back(sets, inputs, y, 0, 0)
    torch.cuda.synchronize()
    n_sent = int(sets[0][1].rank_token_offsets[-1].item())   # partial rows written
    want = [sets[0][0].combined.clone(), sets[0][1].send_row.clone(),
            sets[0][1].partial[:n_sent].clone()]
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bench.pipelined(torch, lambda i, s: bench.hierarchical_front(w, sets, inputs, i, s),
                        lambda i, s: bench.hierarchical_back(sets, inputs, y, i, s),
                        2 * group, steps, side, group)
    for rep in range(2):
        for lb, rb in sets:
            lb.combined.fill_(-7)
            rb.send_row.fill_(-7)
            rb.partial.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for lb, rb in sets:
            assert torch.equal(lb.combined, want[0]), rep
            assert torch.equal(rb.send_row, want[1]), rep
            assert torch.equal(rb.partial[:n_sent], want[2]), rep
    say("  pipelined hierarchical graph replays equal the serial step")
