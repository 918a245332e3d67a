"""The benchmark's pipelined steps (the route and layout of a group of steps,
batched, on a side stream beside the dispatch and combine of the group before, 2 *
group sets of routing and layout buffers in turn, one shared set of row
buffers) give the same results as the same steps run one after the other:
eager, and captured in a HIP graph and replayed. Every step has its own
inputs, so a step that read another step's layout would be caught; each set
ends with the layout of the last step that used it, and the shared row
buffers with the last step's rows and output."""

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

SMALL = ("topk_idx", "topk_weights", "dst_row", "src_pair", "expert_counts", "expert_offsets",
         "rank_counts", "rank_token_counts", "overflow")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    M.lib()
    yield
    torch.cuda.synchronize()


def _small(b):
    return {n: getattr(b, n).clone() for n in SMALL}


def _rows(b):
    live = b.src_pair >= 0
    out = {"rows": b.dispatched[live].clone(), "combined": b.combined.clone()}
    if b.scales is not None:
        out["scales"] = b.scales[live].clone()
    return out


def _poison(sets):
    for b in sets:
        for n in SMALL:
            v = getattr(b, n)
            v.fill_(-7.0 if v.dtype == torch.float32 else -7)
    sets[0].dispatched.fill_(0x55)
    sets[0].combined.fill_(-7)


def _check(sets, want_small, want_rows, what):
    steps = len(want_small)
    for i in range(max(0, steps - len(sets)), steps):      # the last user of each set
        for n, v in want_small[i].items():
            assert torch.equal(getattr(sets[i % len(sets)], n), v), (what, i, n)
    last = sets[(steps - 1) % len(sets)]
    for n, v in want_rows.items():
        got = _rows(last)[n]
        assert torch.equal(got, v), (what, "rows of the last step", n)


@pytest.mark.parametrize("name,steps,group,lead", [
    ("dsv3", 10, 4, 4), ("dsv3", 5, 1, 1), ("decode", 11, 4, 4),
    # the bench's shape: groups of 16 after a first group of 8, fronts in batched calls of 8
    ("dsv3", 21, 16, 8), ("decode", 40, 16, 8)])
def test_pipelined_steps_equal_serial_steps(name, steps, group, lead):
    w = W.WORKLOADS[name]
    say("pipelined steps", name, "x", steps, "in groups of", group, "after a first of", lead)
    seeds = [w.step_seed0 + i for i in range(steps)] if w.steps > 1 else list(range(steps))
    inputs = []
    for s in seeds:
        inp = W.make_inputs(w, s)
        inputs.append(dict(logits=dev(inp.logits),
                           bias=dev(inp.bias) if inp.bias is not None else None,
                           x=dev(inp.x)))
    base = M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                   dtype=w.dispatch_dtype)
    sets = [base] + [base.sharing_rows() for _ in range(2 * group - 1)]
    g = np.random.Generator(np.random.PCG64(3))
    y = dev(W.random_bf16_rows(g, base.num_rows, w.hidden))

    # serial reference: every step alone in its own buffers
    ref = M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                  dtype=w.dispatch_dtype)
    want_small, want_rows = [], None
    for i in range(steps):
        bench.serial_steps(w, [ref], inputs, y, i, 1)
        torch.cuda.synchronize()
        want_small.append(_small(ref))
    want_rows = _rows(ref)
    # the serial form with separate layout and dispatch launches gives the same
    alt = M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                  dtype=w.dispatch_dtype)
    bench.serial_steps(w, [alt], inputs, y, 0, steps, fuse=False)
    torch.cuda.synchronize()
    for n, v in want_small[-1].items():
        assert torch.equal(getattr(alt, n), v), ("unfused serial", n)
    for n, v in _rows(alt).items():
        assert torch.equal(v, want_rows[n]), ("unfused serial rows", n)

    side = torch.cuda.Stream()
    _poison(sets)
    bench.overlapped_steps(torch, w, sets, inputs, y, 0, steps, side, group, lead)
    torch.cuda.synchronize()
    _check(sets, want_small, want_rows, "eager")
    say("  eager pipelined steps equal the serial ones")

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        bench.overlapped_steps(torch, w, sets, inputs, y, 0, steps, side, group, lead)
    for rep in range(2):
        _poison(sets)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(sets, want_small, want_rows, "graph %d" % rep)
    say("  graph replays equal the serial steps")


@pytest.mark.parametrize("group,lead,steps", [(2, 2, 5), (16, 8, 21)])
def test_pipelined_hierarchical_steps_equal_serial_steps(group, lead, steps):
    """The hierarchical pass pipelined the same way (route, expert layout and
    (token, rank) layout of a group beside the send, fan-out and combines of
    the group before; the bench's shape is groups of 16 after a first group
    of 8, fronts in batched calls of 8), replayed from a graph, against the
    same steps run one after the other: each set's (token, rank) layout of
    the last step that used it, and the last step's partials and output."""
    w = W.WORKLOADS["dsv3"]
    say("pipelined hierarchical steps x", steps, "in groups of", group, "after a first of", lead)
    inputs = []
    for s in range(steps):
        inp = W.make_inputs(w, 10 + s)
        inputs.append(dict(logits=dev(inp.logits), bias=dev(inp.bias), x=dev(inp.x)))
    lb0 = M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, 0,
                                  dtype=w.dispatch_dtype)
    rb0 = M.RankBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks,
                                 dtype=w.dispatch_dtype)
    sets = [(lb0, rb0)] + [(lb0.sharing_rows(), rb0.sharing_rows()) for _ in range(2 * group - 1)]
    g = np.random.Generator(np.random.PCG64(4))
    y = dev(W.random_bf16_rows(g, lb0.num_rows, w.hidden))
    ref = [(M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, 0,
                                    dtype=w.dispatch_dtype),
            M.RankBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks,
                                   dtype=w.dispatch_dtype))]
    want_send = []
    for i in range(steps):
        bench.hierarchical_front(w, ref, inputs, i, 0)
        bench.hierarchical_back(ref, inputs, y, i, 0)
        torch.cuda.synchronize()
        want_send.append(ref[0][1].send_row.clone())
    n_sent = int(ref[0][1].rank_token_offsets[-1].item())   # partial rows of the last step
    want = [ref[0][0].combined.clone(), ref[0][1].partial[:n_sent].clone()]
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bench.pipelined(torch, lambda pairs: bench.hierarchical_fronts(w, sets, inputs, pairs),
                        lambda i, s: bench.hierarchical_back(sets, inputs, y, i, s),
                        2 * group, steps, side, group, lead)
    for rep in range(2):
        for lb, rb in sets:
            rb.send_row.fill_(-7)
        lb0.combined.fill_(-7)
        rb0.partial.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(max(0, steps - 2 * group), steps):      # the last user of each set
            assert torch.equal(sets[i % (2 * group)][1].send_row, want_send[i]), (rep, i)
        assert torch.equal(lb0.combined, want[0]), rep
        assert torch.equal(rb0.partial[:n_sent], want[1]), rep
    say("  pipelined hierarchical graph replays equal the serial steps")
