"""moe_layout_no_alloc (the layout with the library's static device scratch)
against moe_layout with a caller's workspace, through the C ABI: every output
bit for bit, on calls in a row whose sizes shrink, so that the second and
later calls run on scratch that still holds a larger earlier call's counts.

The cases cover the scan pass (many tiles: 65,536 tokens at E = 256, k = 8,
1 MiB of per-tile counts), the DeepSeek-V3-shaped layer, capacity mode with
drops, a single tile, and an empty call."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import combine_moe_layout_06_amd as M  # noqa: E402
from synth import workloads as W  # noqa: E402

OUTPUTS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
           "rank_token_counts", "dst_row", "src_pair", "overflow")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _buffers(t, e, k, r, cap):
    rows = e * cap if cap > 0 else t * k
    shapes = dict(expert_counts=e, expert_offsets=e + 1, rank_counts=r, rank_offsets=r + 1,
                  rank_token_counts=r, dst_row=max(t * k, 1), src_pair=max(rows, 1),
                  overflow=1)
    out = {}
    for name, n in shapes.items():
        b = torch.empty(n, dtype=torch.int32, device="cuda")
        b.view(torch.uint8).fill_(0xA5)            # poison: every read value must be written
        out[name] = b
    return out


def _run(fn, t, e, k, r, cap, idx_dev):
    b = _buffers(t, e, k, r, cap)
    args = [t, e, k, r, cap, idx_dev] + [b[n] for n in OUTPUTS]
    if fn == "ws":
        nbytes = M.moe_layout_workspace_bytes(t, e, k)
        ws = torch.empty(max(nbytes, 4), dtype=torch.uint8, device="cuda")
        M.moe_layout(*args, ws, nbytes)
    else:
        M.moe_layout_no_alloc(*args)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy() for n, v in b.items()}


CALLS = [
    # T, E, k, R, cap, mask_frac
    (65536, 256, 8, 32, 0, 0.0),     # scan pass over 512 tiles
    (4096, 256, 8, 32, 0, 0.0),      # DeepSeek-V3-shaped layer
    (3000, 64, 4, 8, 150, 0.05),     # capacity mode with drops
    (100, 8, 2, 4, 0, 0.1),          # one tile
    (0, 8, 2, 4, 0, 0.0),            # empty
]


def test_no_alloc_layout_equals_moe_layout_on_shrinking_calls():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    M.lib()
    for i, (t, e, k, r, cap, mf) in enumerate(CALLS):
        say("no-alloc layout call %d: T=%d E=%d k=%d R=%d cap=%d" % (i, t, e, k, r, cap))
        assert M.moe_layout_workspace_bytes(t, e, k) <= 2 << 20
        g = W.rng(1000 + i)
        idx = W.random_topk_idx(g, t, e, k, mask_frac=mf)
        idx_dev = torch.from_numpy(idx if t else np.zeros((1, k), np.int32)).cuda()
        want = _run("ws", t, e, k, r, cap, idx_dev)
        got = _run("no_alloc", t, e, k, r, cap, idx_dev)
        rows = e * cap if cap > 0 else t * k
        for n in OUTPUTS:
            m = {"dst_row": t * k, "src_pair": rows}.get(n, want[n].size)
            assert np.array_equal(got[n][:m], want[n][:m]), (i, n)
        if t:
            assert int(got["expert_counts"].sum()) == int((idx >= 0).sum())
