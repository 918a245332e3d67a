#!/usr/bin/env python3
"""Throughput of the MoE expert-parallel hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
route (group-limited sigmoid top-k) -> layout (counts, offsets, stable
rows) -> dispatch (FP8 e4m3 + per-1x128 scales) -> combine (weighted bf16
sum). Layout and dispatch go through moe_layout_dispatch, which is one
launch for decode-sized inputs in capacity mode and the two launches
otherwise. The stand-in expert between dispatch and combine is not part of the
path: its output (dequantised rows) is prepared once before timing.

Default workload: the DeepSeek-V3-shaped layer, T=4096 tokens, hidden 7168,
256 experts in 8 groups (top-4 groups, top-8 experts), 32 simulated ranks,
FP8 dispatch, bf16 combine. Inputs are seeded synthetic data already resident
in HBM when timing starts. The timed steps are captured once into a HIP graph
and replayed (every kernel of every step still runs; the host only stops
issuing the launches one by one); --eager launches them from the host instead.
Steps are independent batches, so by default they are pipelined on two
streams in groups of 16 steps after a first group of 8 (pipe_shape): the
routes and layouts of one group (batched
launches) run beside the dispatch and combine of the group before, on 2 *
group sets of routing and layout buffers used in turn (--serial: one step
after the other; the default with --eager). The serial rate of the same steps
is measured in the same run and reported beside it.

Prints one JSON line. Besides the contract fields it carries:
  roofline      HBM roofline of the dominant kernel (combine): algorithmic
                bytes per launch / average launch time, from HIP events on
                the launch stream around 20 back-to-back launches (no event
                between launches, so it matches the profiler's kernel time);
                `traffic` comes from the committed rocprofv3 counter summary
                when it was taken on the current kernel source, else null
  cpu_baseline  the CPU oracle (numpy) timed on this host: all host cores
                (worker processes over token ranges; the headline value) and
                one thread on the first 256 tokens, each split into route,
                layout + dispatch and combine, median of 5 passes
  phases_us     average per-phase times from HIP events, taken in a second
                pass over the same steps (the timed loop itself has no events)
  cold_us_per_step  the same step with a 1 GiB write between steps, which
                evicts L2 and the 256 MB Infinity Cache
  serial_ms_per_step  the timed steps run one after the other on one stream
  event_us_per_step_median/_p99  per-step times of the event pass (steps one
                after the other, an event between phases)
  pipelined_stamps  latency (route start to combine end) and interval (between
                combine ends) percentiles of pipelined steps, from wall-clock
                stamp kernels in a separate replay
  ceilings_gbps best GB/s of plain kernels (libmoe_ceilings.so) with the
                path's access patterns: sequential copy, read and write, and
                random whole-row gather (combine-like) and scatter
                (dispatch-like); copy_ceiling_gbps is the sequential copy
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_dsv3_traffic.json")
COMBINE_SOURCES = [os.path.join(ROOT, "combine_moe_layout_06_amd", "csrc", f)
                   for f in ("combine.hip", "wave.h", "kernels.h")]
HIER_SOURCES = [os.path.join(ROOT, "combine_moe_layout_06_amd", "csrc", f)
                for f in ("hierarchical.hip", "wave.h", "kernels.h")]
# counter records of the other passes' roofline kernels (combine_local, combine_backward)
KERNEL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "roofline_traffic.json")
ROOF_REPS = 20   # back-to-back launches timed for the roofline kernel


def launch_us(torch, fn, reps=ROOF_REPS):
    """Average duration of one launch of `fn`: HIP events on the current
    (launch) stream around `reps` back-to-back launches, so that no event
    sits between two launches."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps * 1e3


def roofline_timing():
    return "HIP events around %d back-to-back launches on the launch stream" % ROOF_REPS


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="dsv3",
                   choices=["dsv3", "mixtral", "qwen3_skew", "tiny", "decode"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--dispatch", default="auto", choices=["auto", "bf16", "fp8", "mxfp8"],
                   help="dispatched format (auto: the workload's own)")
    p.add_argument("--cold-steps", type=int, default=10)
    g = p.add_mutually_exclusive_group()
    g.add_argument("--graph", dest="graph", action="store_true", default=True,
                   help="capture the timed steps into one HIP graph and replay it (default)")
    g.add_argument("--eager", dest="graph", action="store_false",
                   help="launch the timed steps one by one from the host instead")
    o = p.add_mutually_exclusive_group()
    o.add_argument("--overlap", dest="overlap", action="store_true", default=None,
                   help="pipeline the steps on two streams: the route and layout of a group "
                        "of steps run beside the dispatch and combine of the group before "
                        "(default with graph replay)")
    o.add_argument("--serial", dest="overlap", action="store_false",
                   help="run each step after the previous one on a single stream (default "
                        "with --eager)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--pass", dest="pass_", default="forward",
                   choices=["forward", "backward", "hierarchical"],
                   help="backward: time combine-backward then dispatch-backward instead; "
                        "hierarchical: one row per (token, rank) out, per-rank partial sums back")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def step_bytes(w, rows_live, dtype=None):
    """Algorithmic bytes of one step, per phase (what the method must move).
    dtype: 0 bf16, 1 FP8 (fp32 scale per 128 columns), 2 MXFP8 (one byte per
    32 columns); defaults to the workload's own."""
    T, H, E, k = w.tokens, w.hidden, w.experts, w.top_k
    rows = w.num_rows
    dtype = w.dispatch_dtype if dtype is None else dtype
    route = T * E * 4 + (E * 4 if w.bias != "none" else 0) + T * k * 8
    layout = T * k * 4 + T * k * 4 + rows * 4 + (3 * E + 3 * w.ranks + 3) * 4
    if dtype == 1:
        dispatch = T * H * 2 + T * k * 4 + rows_live * H + rows_live * (H // 128) * 4
    elif dtype == 2:
        dispatch = T * H * 2 + T * k * 4 + rows_live * H + rows_live * (H // 32)
    else:
        dispatch = T * H * 2 + T * k * 4 + rows_live * H * 2
    combine = rows_live * H * 2 + T * k * 8 + T * H * 2
    return dict(route=route, layout=layout, dispatch=dispatch, combine=combine)


def backward_bytes(w, rows_live):
    """Algorithmic bytes of the backward pair: combine-backward reads dout,
    the expert rows, dst_row and weights and writes the row gradients and
    the weight gradients; dispatch-backward reads the row gradients and
    dst_row and writes dx."""
    T, H, k = w.tokens, w.hidden, w.top_k
    combine_bwd = T * H * 2 + rows_live * H * 2 + T * k * 8 + rows_live * H * 2 + T * k * 4
    dispatch_bwd = rows_live * H * 2 + T * k * 4 + T * H * 2
    return dict(combine_backward=combine_bwd, dispatch_backward=dispatch_bwd)


def run_backward(args, w, M, W, torch, np):
    """Backward pair on the layout of one forward pass: combine-backward
    (dout, expert rows -> row gradients, weight gradients), then
    dispatch-backward (row gradients -> dx)."""
    dev = torch.device("cuda:0")
    inp = W.make_inputs(w, args.seed)
    buf = M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                  device=dev)
    bias = torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None
    buf.route(torch.from_numpy(inp.logits).to(dev), bias, w.score_fn, w.groups, w.topk_groups)
    buf.layout()
    rows = buf.num_rows
    g = W.rng(args.seed + 1)
    y = torch.from_numpy(W.random_bf16_rows(g, rows, w.hidden).view(np.int16)).to(dev)
    dout = torch.from_numpy(W.random_bf16_rows(g, w.tokens, w.hidden).view(np.int16)).to(dev)
    dy = torch.empty_like(y)
    dw = torch.empty((w.tokens, w.top_k), dtype=torch.float32, device=dev)
    dx = torch.empty((w.tokens, w.hidden), dtype=torch.int16, device=dev)
    T, H, k = w.tokens, w.hidden, w.top_k

    def step():
        M.moe_combine_backward(T, H, k, rows, dout, y, buf.dst_row, buf.topk_weights, dy, dw)
        M.moe_dispatch_backward(T, H, k, rows, dy, buf.dst_row, dx)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evict_caches(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record()
        M.moe_combine_backward(T, H, k, rows, dout, y, buf.dst_row, buf.topk_weights, dy, dw)
        e[1].record()
        M.moe_dispatch_backward(T, H, k, rows, dy, buf.dst_row, dx)
        e[2].record()
    torch.cuda.synchronize()
    cb = sum(e[0].elapsed_time(e[1]) for e in ev) / len(ev) * 1e-3
    db = sum(e[1].elapsed_time(e[2]) for e in ev) / len(ev) * 1e-3
    rows_live = int((buf.dst_row >= 0).sum().item())
    nb = backward_bytes(w, rows_live)
    ms = wall * 1e3 / args.steps
    total = sum(nb.values())
    cb_us = launch_us(torch, lambda: M.moe_combine_backward(T, H, k, rows, dout, y, buf.dst_row,
                                                             buf.topk_weights, dy, dw))
    achieved = nb["combine_backward"] / (cb_us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "backward dispatch+combine tokens/s and HBM GB/s, %s shape, 1 GPU" % w.name,
        "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s backward: T=%d H=%d E=%d k=%d, bf16 gradients"
                   % (w.name, T, H, w.experts, k), "tokens": T, "hidden": H, "top_k": k},
        "gbps": round(total / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total, "phase_bytes": nb,
        "phases_us": {"combine_backward": round(cb * 1e6, 2), "dispatch_backward": round(db * 1e6, 2)},
        "cache_eviction": EVICTION,
        "roofline": {"bound": "hbm", "kernel": "combine_backward", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_kernel_traffic("combine_backward", COMBINE_SOURCES,
                                                    nb["combine_backward"]),
                     "algorithmic_bytes_per_launch": nb["combine_backward"],
                     "launch_us": round(cb_us, 2), "timing": roofline_timing()},
        "cpu_baseline": None}), flush=True)


def scale_bytes(H, dtype):
    return {0: 0, 1: (H // 128) * 4, 2: H // 32}[dtype]


def hierarchical_bytes(w, rows_live, n_sent, dtype):
    """Algorithmic bytes of the hierarchical pass, per phase. n_sent is the
    number of (token, rank) rows; a fanned-out row is read once per rank row
    it comes from and written once per expert row."""
    T, H, E, k, R = w.tokens, w.hidden, w.experts, w.top_k, w.ranks
    row = (H if dtype else 2 * H) + scale_bytes(H, dtype)
    nrr = T * min(k, R)
    b = step_bytes(w, rows_live, dtype)
    return dict(
        route=b["route"], layout=b["layout"],
        rank_layout=T * k * 4 + 2 * T * k * 4 + nrr * 4 + (2 * R + 1) * 4,
        dispatch=T * H * 2 + T * k * 4 + n_sent * row,
        expand=w.num_rows * 4 + rows_live * 4 + n_sent * row + rows_live * row,
        combine_local=rows_live * H * 2 + T * k * 12 + n_sent * H * 2,
        combine_partials=n_sent * H * 2 + T * k * 4 + T * H * 2)


def hierarchical_front(w, sets, inputs, i, s):
    """The latency-bound front of hierarchical step i on buffer set s (a
    LayerBuffers, RankBuffers pair): route, expert layout, (token, rank)
    layout."""
    d = inputs[i % len(inputs)]
    lb, rb = sets[s]
    lb.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups)
    lb.layout()
    rb.rank_layout(lb.topk_idx)


def _moe():
    import combine_moe_layout_06_amd as M
    return M


def hierarchical_fronts(w, sets, inputs, pairs):
    """hierarchical_front of steps (i, s) in `pairs`: their routes in one
    launch, their expert layouts and their (token, rank) layouts in one
    launch per pass (the batched entry points), in calls of up to
    MOE_MAX_BATCHES steps."""
    M = _moe()
    for c in range(0, len(pairs), M.MOE_MAX_BATCHES):
        lbs = [sets[s][0] for _, s in pairs[c:c + M.MOE_MAX_BATCHES]]
        rbs = [sets[s][1] for _, s in pairs[c:c + M.MOE_MAX_BATCHES]]
        ds = [inputs[i % len(inputs)] for i, _ in pairs[c:c + M.MOE_MAX_BATCHES]]
        M.route_batches(lbs, [d["logits"] for d in ds], [d["bias"] for d in ds], w.score_fn,
                        w.groups, w.topk_groups)
        M.layout_batches(lbs)
        M.rank_layout_batches(rbs, [lb.topk_idx for lb in lbs])


def hierarchical_back(sets, inputs, y, i, s):
    """The rest of hierarchical step i: one copy per (token, rank), fan-out
    to the expert rows, per-(token, rank) partial sums of the expert outputs
    y, and the per-token sum."""
    d = inputs[i % len(inputs)]
    lb, rb = sets[s]
    rb.dispatch(d["x"])
    rb.expand(lb)
    rb.combine_local(lb, y)
    rb.combine_partials(lb.combined)


def run_hierarchical(args, w, M, W, torch, np):
    """Deduplicated dispatch and hierarchical combine: route, expert layout,
    (token, rank) layout, one copy per (token, rank), fan-out to the expert
    rows, then per-(token, rank) partial sums and the per-token sum."""
    dev = torch.device("cuda:0")
    dtype = {"auto": w.dispatch_dtype, "bf16": 0, "fp8": 1, "mxfp8": 2}[args.dispatch]
    T, H, k = w.tokens, w.hidden, w.top_k
    n_inputs = args.steps + args.warmup if w.steps > 1 else 1
    seeds = [w.step_seed0 + i for i in range(n_inputs)] if w.steps > 1 else [args.seed]
    inputs = []
    for s in seeds:
        inp = W.make_inputs(w, s)
        inputs.append(dict(
            logits=torch.from_numpy(inp.logits).to(dev),
            bias=torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None,
            x=torch.from_numpy(inp.x.view(np.int16)).to(dev)))
    overlap = args.graph if args.overlap is None else args.overlap
    lb = M.LayerBuffers.allocate(T, H, w.experts, k, w.ranks, w.capacity, device=dev,
                                 dtype=dtype)
    rb = M.RankBuffers.allocate(T, H, w.experts, k, w.ranks, dtype=dtype, device=dev)
    # pipelined steps: 2 * group sets of layout buffers in turn, row buffers
    # shared
    group, lead = pipe_shape(w)
    nsets = 2 * group if overlap else 1
    sets = [(lb, rb)] + [(lb.sharing_rows(), rb.sharing_rows()) for _ in range(nsets - 1)]

    phases = ["route", "layout", "rank_layout", "dispatch", "expand", "combine_local",
              "combine_partials"]

    def calls(i):
        d = inputs[i % len(inputs)]
        return [lambda: lb.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups),
                lb.layout, lambda: rb.rank_layout(lb.topk_idx), lambda: rb.dispatch(d["x"]),
                lambda: rb.expand(lb), lambda: rb.combine_local(lb, y),
                lambda: rb.combine_partials(lb.combined)]

    def front(i, s):
        hierarchical_front(w, sets, inputs, i, s)

    def back(i, s):
        hierarchical_back(sets, inputs, y, i, s)

    def serial(first, n):
        for i in range(first, first + n):
            front(i, 0)
            back(i, 0)

    def piped(first, n):
        pipelined(torch, lambda pairs: hierarchical_fronts(w, sets, inputs,
                                                           [(first + i, s) for i, s in pairs]),
                  lambda i, s: back(first + i, s), nsets, n, side, group, lead)

    side = torch.cuda.Stream() if overlap else None

    # stand-in expert output: the fanned-out rows of step 0, dequantised
    y = None
    for c in calls(0)[:5]:
        c()
    torch.cuda.synchronize()
    rows = lb.num_rows
    if dtype == 1:
        codes = lb.dispatched[:rows].view(torch.float8_e4m3fn).float()
        y = (codes * lb.scales[:rows].repeat_interleave(128, dim=1)).to(torch.bfloat16)
    elif dtype == 2:
        codes = lb.dispatched[:rows].view(torch.float8_e4m3fn).float()
        sc = torch.exp2(lb.scales[:rows].float() - 127.0).repeat_interleave(32, dim=1)
        y = (codes * sc).to(torch.bfloat16)
    else:
        y = lb.dispatched[:rows].view(torch.bfloat16).clone()
    y = y.view(torch.int16).contiguous()
    rows_live = int((lb.dst_row >= 0).sum().item())
    n_sent = int(rb.rank_token_offsets[-1].item())

    serial(0, args.warmup)
    if overlap:
        piped(0, args.warmup)
    torch.cuda.synchronize()
    serial_wall = timed_run(torch, lambda: serial(args.warmup, args.steps), args.graph)
    wall = (timed_run(torch, lambda: piped(args.warmup, args.steps), args.graph)
            if overlap else serial_wall)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        for j, c in enumerate(calls(args.warmup + i)):
            c()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    ph = {n: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / len(ev) * 1e3
          for j, n in enumerate(phases)}
    nb = hierarchical_bytes(w, rows_live, n_sent, dtype)
    ms = wall * 1e3 / args.steps
    total = sum(nb.values())
    dom = max(("dispatch", "expand", "combine_local", "combine_partials"), key=lambda n: ph[n])
    dom_us = launch_us(torch, calls(args.warmup)[phases.index(dom)])
    achieved = nb[dom] / (dom_us * 1e-6) / 1e9
    row = (H if dtype else 2 * H) + scale_bytes(H, dtype)
    out = {
        "metric": "hierarchical dispatch+combine tokens/s, %s shape, 1 GPU" % w.name,
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {0: "bf16", 1: "fp8e4m3+bf16", 2: "mxfp8e4m3+bf16"}[dtype],
        "data": "synthetic",
        "launch": ("hip graph replay" if args.graph else "eager launches") +
                  ("; steps pipelined on two streams in groups of %d (the first of %d): the "
                   "route, expert layout and (token, rank) layout of one group run beside "
                   "the send, fan-out and combines of the group before (%d sets of layout "
                   "buffers in turn, row buffers shared)"
                   % (group, min(lead, group), 2 * group) if overlap
                   else "; one step after the other on one stream"),
        "serial_ms_per_step": round(serial_wall * 1e3 / args.steps, 5),
        "cache_eviction": EVICTION,
        "config": {"workload": "%s hierarchical: T=%d H=%d E=%d k=%d R=%d, one row per "
                   "(token, rank), bf16 partials" % (w.name, T, H, w.experts, k, w.ranks),
                   "tokens": T, "hidden": H, "experts": w.experts, "top_k": k,
                   "ranks": w.ranks, "seed": args.seed},
        "gbps": round(total / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total, "phase_bytes": nb,
        "phases_us": {n: round(v, 2) for n, v in ph.items()},
        "rows": {"pairs": rows_live, "sent": n_sent},
        "exchanged_bytes": {"flat": rows_live * row + rows_live * H * 2,
                            "hierarchical": n_sent * row + n_sent * H * 2},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_kernel_traffic(dom, HIER_SOURCES, nb[dom]),
                     "algorithmic_bytes_per_launch": nb[dom],
                     "launch_us": round(dom_us, 2), "timing": roofline_timing()},
        "cpu_baseline": None}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_hierarchical(w, args.seed, args.cpu_seconds, dtype)
    print(json.dumps(out), flush=True)


def cpu_baseline_hierarchical(w, seed, budget_s, dtype):
    """The CPU oracle of the hierarchical pass on the first 512 tokens."""
    from oracle import moe_oracle as O
    from synth import workloads as W

    ts = min(w.tokens, 512)
    inp = W.make_inputs(w, seed, tokens=ts)
    disp = {0: O.dispatch_bf16, 1: O.dispatch_fp8, 2: O.dispatch_mxfp8}[dtype]
    idx, wt = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    L = O.layout(idx, w.experts, w.ranks, w.capacity)
    y, _ = O.dispatch_bf16(inp.x, L["dst_row"], L["num_rows"])
    reps, t0 = 0, time.perf_counter()
    while True:
        idx, wt = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
        L = O.layout(idx, w.experts, w.ranks, w.capacity)
        rl = O.rank_layout(idx, w.experts, w.ranks)
        sent = disp(inp.x, rl["send_row"], rl["num_rank_rows"])
        for part in sent[:-1]:
            O.expand_rows(part, rl["rank_row"], L["src_pair"])
        O.combine_hierarchical(y, L["dst_row"], wt, rl)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": ts * reps / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%s shape, first %d of %d tokens, %d repeats of the hierarchical pass "
                      "in %.1f s (numpy, single thread)" % (w.name, ts, w.tokens, reps, el)}


def code_only(text):
    """C/C++ source text without comments and whitespace, so that edits to
    comments or layout leave the source hash unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return "".join(text.split())


def sha_of(paths):
    """SHA-256 over the code (comments and whitespace removed) of `paths`."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()


def load_traffic(algorithmic_bytes):
    """HBM bytes per combine launch from the committed counter summary, or
    None when it is missing, was taken on a different kernel source, or on
    a different workload (its algorithmic bytes differ)."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != sha_of(COMBINE_SOURCES):
        return None
    if d.get("algorithmic_bytes_per_launch") != algorithmic_bytes:
        return None
    return d.get("traffic_bytes_per_launch")


def load_kernel_traffic(kernel, sources, algorithmic_bytes):
    """HBM bytes per call of `kernel` from the committed counter records, or
    None when there is no record of it taken on the current source of
    `sources` for a workload with these algorithmic bytes."""
    try:
        with open(KERNEL_TRAFFIC_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    sha = sha_of(sources)
    for d in recs if isinstance(recs, list) else []:
        if (d.get("kernel") == kernel and d.get("kernel_source_sha256") == sha
                and d.get("algorithmic_bytes_per_launch") == algorithmic_bytes):
            return d.get("traffic_bytes_per_launch")
    return None


def calibrate_copy():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 5}), flush=True)


CEIL_LIB = os.path.join(ROOT, "combine_moe_layout_06_amd", "libmoe_ceilings.so")
CEIL_BYTES = 1 << 30     # sequential probes: 1 GiB read and/or written
CEIL_REPS = 10


_measure_lib = None


def measure_lib():
    """libmoe_ceilings.so with its argument types (ceiling kernels, stamps)."""
    global _measure_lib
    if _measure_lib is None:
        import ctypes

        if not os.path.exists(CEIL_LIB):
            raise RuntimeError("%s is missing; run `python -m combine_moe_layout_06_amd.build`"
                               % CEIL_LIB)
        L = ctypes.CDLL(CEIL_LIB)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.ceil_copy.argtypes = [vp, vp, sz, i32, i32, i32, vp]
        L.ceil_read.argtypes = [vp, sz, vp, i32, i32, i32, vp]
        L.ceil_write.argtypes = [vp, sz, i32, i32, i32, vp]
        L.ceil_rows.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, vp]
        L.ceil_fanout.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.bench_stamp.argtypes = [vp, i32, vp]
        L.ceil_rows_one_way.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, vp, vp]
        L.ceil_rows_one_way.restype = i32
        for f in (L.ceil_copy, L.ceil_read, L.ceil_write, L.ceil_rows, L.ceil_fanout,
                  L.bench_stamp):
            f.restype = i32
        L.bench_stamp_hz.argtypes = []
        L.bench_stamp_hz.restype = ctypes.c_double
        _measure_lib = L
    return _measure_lib


def stamped_pipeline(torch, np, front, back, nsets, steps, side, group, lead):
    """Per-step latency and completion intervals of pipelined steps, from
    the GPU's wall clock: the pipelined steps are captured again with a
    one-wave stamp kernel before each step's front (on the side stream) and
    after each step's back (on the current stream), replayed
    GRAPH_WARM_REPLAYS times, then once for the stamps. The stamps add two
    small kernels per step, so this pass is separate from the timed one and
    reports its own us/step beside the percentiles."""
    L = measure_lib()
    hz = L.bench_stamp_hz()
    if hz <= 0:
        return None
    st = torch.zeros((2, steps), dtype=torch.int64, device="cuda")

    def stamp(slot):
        rc = L.bench_stamp(st.data_ptr(), slot, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError("bench_stamp failed: %d" % rc)

    def f(pairs):
        for i, _ in pairs:
            stamp(i)
        front(pairs)

    def b(i, s):
        back(i, s)
        stamp(steps + i)

    wall = timed_run(torch, lambda: pipelined(torch, f, b, nsets, steps, side, group, lead),
                     True)
    t = st.cpu().numpy().astype(np.float64) * 1e6 / hz       # microseconds
    lat = t[1] - t[0]
    gap = np.diff(t[1])
    pct = lambda a, q: round(float(np.percentile(a, q)), 2)
    first = float(lat[0] - (np.median(gap) if len(gap) else 0.0))
    return {"us_per_step": round(wall * 1e6 / steps, 2),
            "latency_us_p50": pct(lat, 50), "latency_us_p99": pct(lat, 99),
            "interval_us_p50": pct(gap, 50), "interval_us_p99": pct(gap, 99),
            "fill_us": round(first, 2),
            "clock_hz": hz,
            "what": "latency: a step's route start to its combine end; interval: between "
                    "consecutive combine ends; fill: the first step's latency minus the median "
                    "interval (the front work nothing hides); one replay of the pipelined steps "
                    "with a stamp kernel before each front and after each back"}


def ceilings(torch, np):
    """Best GB/s of plain kernels with the path's access patterns on this GPU
    (libmoe_ceilings.so), each over a small sweep of launch shapes; HIP events
    on the launch stream around CEIL_REPS back-to-back launches:
      copy     sequential 16-byte reads + writes (bytes read + written)
      read     sequential reads only
      write    sequential writes only
      gather   random whole-row reads of 14,336-byte rows (bf16 rows of the
               DeepSeek-V3 shape), sequential writes (read + written)
      scatter  sequential reads, random whole-row writes of 7,168-byte rows
               (its FP8 rows) (read + written)
      fanout   each 7,168-byte row read once and written to 8 random rows
               (the dispatch's pattern at k = 8) (read + written)
      shuffle  random whole-row reads and random whole-row writes of 14,336-
               byte rows (the backward pair's and the partial combine's mix)
      rread    random whole-row reads of 14,336-byte rows, nothing written
      rwrite   random whole-row writes of 7,168-byte rows, nothing read"""
    L = measure_lib()

    n = CEIL_BYTES
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.fill_(2)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def best(moved, configs, launch):
        top = None
        for cfg in configs:
            def go():
                rc = launch(*cfg)
                if rc != 0:
                    raise RuntimeError("ceiling kernel %s failed: %d" % (cfg, rc))
            go()
            go()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            for _ in range(CEIL_REPS):
                go()
            e.record()
            torch.cuda.synchronize()
            gbps = moved * CEIL_REPS / (s.elapsed_time(e) * 1e-3) / 1e9
            if top is None or gbps > top[0]:
                top = (gbps, cfg)
        return top

    seq = [(pc, u) for pc in (1, 2, 4, 8) for u in (1, 4)]
    out = {}
    g, c = best(2 * n, seq, lambda pc, u: L.ceil_copy(a.data_ptr(), b.data_ptr(), n, cus * pc,
                                                         pc, u, stream))
    out["copy"] = {"gbps": round(g, 1), "per_cu": c[0], "unroll": c[1]}
    g, c = best(n, seq, lambda pc, u: L.ceil_read(a.data_ptr(), n, sink.data_ptr(), cus * pc,
                                                     pc, u, stream))
    out["read"] = {"gbps": round(g, 1), "per_cu": c[0], "unroll": c[1]}
    g, c = best(n, seq, lambda pc, u: L.ceil_write(b.data_ptr(), n, cus * pc, pc, u, stream))
    out["write"] = {"gbps": round(g, 1), "per_cu": c[0], "unroll": c[1]}
    gen = np.random.Generator(np.random.PCG64(12345))
    for name, gather, row_bytes, pieces in (("gather", 1, 14336, (128, 448, 896)),
                                            ("scatter", 0, 7168, (64, 128, 448)),
                                            ("shuffle", 2, 14336, (128, 256, 896))):
        rows = n // row_bytes
        perm = torch.from_numpy(gen.permutation(rows).astype(np.int32)).cuda()
        cfgs = [(p, pc) for p in pieces for pc in (0, 1, 2, 3, 4, 5, 6)]
        g, c = best(2 * rows * row_bytes, cfgs,
                    lambda p, pc: L.ceil_rows(gather, a.data_ptr(), b.data_ptr(),
                                              perm.data_ptr(), rows, row_bytes, p, pc, stream))
        out[name] = {"gbps": round(g, 1), "row_bytes": row_bytes, "piece_bytes": 16 * c[0],
                     "per_cu": c[1]}
    for name, mode, row_bytes, pieces in (("rread", 0, 14336, (128, 448, 896)),
                                          ("rwrite", 1, 7168, (64, 448))):
        rows = n // row_bytes
        perm = torch.from_numpy(gen.permutation(rows).astype(np.int32)).cuda()
        cfgs = [(p, pc) for p in pieces for pc in (0, 2, 3, 4, 5, 6)]
        g, c = best(rows * row_bytes, cfgs,
                    lambda p, pc: L.ceil_rows_one_way(mode, a.data_ptr(), b.data_ptr(),
                                                      perm.data_ptr(), rows, row_bytes, p, pc,
                                                      sink.data_ptr(), stream))
        out[name] = {"gbps": round(g, 1), "row_bytes": row_bytes, "piece_bytes": 16 * c[0],
                     "per_cu": c[1]}
    row_bytes, k = 7168, 8
    rows = n // (row_bytes * k)
    perm = torch.from_numpy(gen.permutation(rows * k).astype(np.int32)).cuda()
    cfgs = [(p, pc) for p in (64, 128, 256, 448) for pc in (0, 1, 2, 3, 4, 5, 6)]
    g, c = best(rows * row_bytes * (1 + k), cfgs,
                lambda p, pc: L.ceil_fanout(a.data_ptr(), b.data_ptr(), perm.data_ptr(), rows, k,
                                            row_bytes, p, pc, stream))
    out["fanout"] = {"gbps": round(g, 1), "row_bytes": row_bytes, "k": k,
                     "piece_bytes": 16 * c[0], "per_cu": c[1]}
    del a, b
    torch.cuda.empty_cache()
    return out


CPU_REPS = 5              # repeats of each CPU-baseline leg (median reported)
CPU_SINGLE_TOKENS = 256   # tokens of the single-thread leg's sample
CPU_MAX_WORKERS = 16      # worker processes at most: the host's CPU share per GPU


def cpu_baseline_phases(w, seed, lo, hi, dtype, reps, barrier=None):
    """The oracle's route, layout + dispatch and combine over tokens [lo, hi)
    of the workload, `reps` times; returns per repeat the seconds of each
    phase. The stand-in expert output is made once, untimed. With a barrier,
    every phase starts when all workers reach it."""
    from oracle import moe_oracle as O
    from synth import workloads as W

    inp = W.make_inputs(w, seed)
    logits, x = inp.logits[lo:hi], inp.x[lo:hi]
    idx, wt = O.route(logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    L = O.layout(idx, w.experts, w.ranks, w.capacity)
    if dtype == 1:
        y_tok = O.expert_dequant(*O.quantize_fp8_blocks(x))
    elif dtype == 2:
        y_tok = O.expert_dequant_mx(*O.quantize_mxfp8_blocks(x))
    else:
        y_tok = x
    y, _ = O.dispatch_bf16(y_tok, L["dst_row"], L["num_rows"])
    disp = {0: O.dispatch_bf16, 1: O.dispatch_fp8, 2: O.dispatch_mxfp8}[dtype]

    def sync():
        if barrier is not None:
            barrier.wait()

    out = []
    for _ in range(reps):
        sync()
        t0 = time.perf_counter()
        idx, wt = O.route(logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
        t1 = time.perf_counter()
        sync()
        t1b = time.perf_counter()
        L = O.layout(idx, w.experts, w.ranks, w.capacity)
        disp(x, L["dst_row"], L["num_rows"])
        t2 = time.perf_counter()
        sync()
        t2b = time.perf_counter()
        O.combine(y, L["dst_row"], wt)
        t3 = time.perf_counter()
        out.append((t1 - t0, t2 - t1b, t3 - t2b))
    return out


def cpu_baseline_worker(name, seed, lo, hi, dtype, reps, barrier, queue):
    """Process body of the all-cores leg: one token range, phases aligned
    with the other workers by the barrier."""
    os.environ["OMP_NUM_THREADS"] = "1"
    from synth import workloads as W
    try:
        queue.put((lo, cpu_baseline_phases(W.WORKLOADS[name], seed, lo, hi, dtype, reps,
                                           barrier)))
    except BaseException as e:  # the parent must not wait forever
        barrier.abort()
        queue.put((lo, repr(e)))


def cpu_baseline(w, seed, dtype=None):
    """The CPU oracle (numpy) on this host, two legs, each split into phases
    (route, layout + dispatch, combine) and timed CPU_REPS times (median):
      single thread: the first CPU_SINGLE_TOKENS tokens of the workload;
      all cores:     the whole workload cut into equal token ranges, one
                     worker process per range, as many as this process may
                     run on (at most CPU_MAX_WORKERS); each phase starts on
                     all workers together and lasts until the slowest ends.
    Must run before anything initialises the GPU in this process: the workers
    are started as new processes. The headline value is the all-cores leg."""
    import multiprocessing as mp

    import numpy as np

    dtype = w.dispatch_dtype if dtype is None else dtype
    names = ("route", "layout_dispatch", "combine")

    def summary(per_rep, tokens):
        ph = np.median(np.asarray(per_rep), axis=0)
        step = float(np.median(np.asarray(per_rep).sum(axis=1)))
        return {"value": round(tokens / step, 1), "tokens": tokens,
                "seconds_per_pass": round(step, 4),
                "phases_s": {n: round(float(v), 4) for n, v in zip(names, ph)}}

    ts = min(w.tokens, CPU_SINGLE_TOKENS)
    single = summary(cpu_baseline_phases(w, seed, 0, ts, dtype, CPU_REPS), ts)

    host_cores = len(os.sched_getaffinity(0))
    n = max(1, min(host_cores, CPU_MAX_WORKERS, w.tokens))
    cuts = [w.tokens * i // n for i in range(n + 1)]
    ctx = mp.get_context("spawn")
    barrier, queue = ctx.Barrier(n, timeout=600), ctx.Queue()
    procs = [ctx.Process(target=cpu_baseline_worker,
                         args=(w.name, seed, cuts[i], cuts[i + 1], dtype, CPU_REPS, barrier,
                               queue)) for i in range(n)]
    for p in procs:
        p.start()
    got = {}
    while len(got) < n:
        try:
            lo, res = queue.get(timeout=5)
            got[lo] = res
        except Exception:   # queue.Empty: stop waiting once a worker is gone
            if any(p.exitcode not in (None, 0) for p in procs):
                barrier.abort()
                for p in procs:
                    p.join(timeout=30)
                raise RuntimeError("cpu_baseline: a worker process exited with code %s"
                                   % [p.exitcode for p in procs])
    for p in procs:
        p.join()
    errors = [v for v in got.values() if isinstance(v, str)]
    if errors:
        raise RuntimeError("cpu_baseline worker failed: %s" % errors[0])
    # per repeat and phase: the slowest worker
    per_rep = np.max(np.stack([np.asarray(got[lo]) for lo in cuts[:-1]]), axis=0)
    allc = summary(per_rep, w.tokens)
    allc["workers"] = n
    return {"value": allc["value"], "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": "%s shape, seed %d: all %d tokens cut into %d token ranges, one numpy "
                      "oracle process per range (host offers %d cores); route, layout+dispatch "
                      "and combine each timed from a common start to the slowest worker; "
                      "median of %d passes" % (w.name, seed, w.tokens, n, host_cores, CPU_REPS),
            "host_cores": host_cores,
            "all_cores": allc,
            "single_thread": dict(single, sample="first %d tokens, one thread" % ts)}


def serial_steps(w, bufs, inputs, y, first, steps, fuse=True):
    """`steps` steps one after the other on the current stream: route,
    layout + dispatch, combine; step i uses the inputs of step first + i.
    fuse: layout and dispatch through moe_layout_dispatch (one launch for
    decode-sized inputs in capacity mode: the fewest launches for steps
    launched from the host), else moe_layout then moe_dispatch (faster from a
    graph, where a launch costs little: decode 17.9 against 19.7 us/step)."""
    b = bufs[0]
    for i in range(steps):
        d = inputs[(first + i) % len(inputs)]
        b.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups)
        if fuse:
            b.layout_dispatch(d["x"])
        else:
            b.layout()
            b.dispatch(d["x"])
        b.combine(y)


PIPE_GROUP = 16   # steps per cross-stream wait of the pipelined mode
PIPE_LEAD = 8     # steps of the first group


def pipe_shape(w):
    """(group, first group) of the pipelined mode. Same process, batched
    fronts: groups of 16 after a first group of 8 ran the DeepSeek-V3-shaped
    steps at 147.2 / 146.5 us/step (20 / 50 steps, median of 10) against 148.4
    / 148.3 in groups of 8, mixtral ~1 us faster, qwen3_skew within noise, and
    decode steps at 11.6 / 11.7 us (50 / 200 steps, median of 8) against 12.1 /
    12.3 in groups of 8."""
    return PIPE_GROUP, PIPE_LEAD


def pipeline_groups(steps, group=PIPE_GROUP, lead=PIPE_LEAD):
    """Groups of the pipelined mode: the first `lead` steps, then groups of
    `group` steps (the last one shorter)."""
    first = min(max(lead, 1), group, steps)
    out = [range(0, first)] if steps else []
    out += [range(g0, min(g0 + group, steps)) for g0 in range(first, steps, group)]
    return out


def pipelined(torch, front, back, nsets, steps, side, group=PIPE_GROUP, lead=PIPE_LEAD):
    """Steps pipelined on two streams, in the groups of pipeline_groups():
    `side` runs front(pairs) (route and layout of the group's steps, pairs =
    [(i, s), ...]) while the current stream runs back(i, s) (dispatch and
    combine) for the steps of the group before; then the current stream
    waits for the side stream once and runs back() for the group. Step i
    uses the routing and layout buffers of set s = i % nsets (nsets = 2 *
    group); the backs share one set of row buffers, used one step after the
    other on the current stream. Two consecutive groups hold at most nsets
    steps, so the steps that last used the sets of group q are in group q - 2
    or earlier: the fronts of group q wait, once, until the backs of group
    q - 2 are done. One event per group in each direction: each cross-stream
    edge costs the stream after it a few microseconds. (Without the release
    waits, with buffers of its own for every step, the side stream could run
    all fronts ahead; replayed, that graph ran decode steps 22% slower and
    dsv3 steps no faster.)"""
    assert nsets == 2 * group
    main = torch.cuda.current_stream()   # the capturing stream inside a graph capture
    released = []
    for _ in range(2):
        e = torch.cuda.Event()
        e.record(main)
        released.append(e)
    for q, grp in enumerate(pipeline_groups(steps, group, lead)):
        side.wait_event(released[q % 2])
        with torch.cuda.stream(side):
            front([(i, i % nsets) for i in grp])
        ready = torch.cuda.Event()
        ready.record(side)
        main.wait_event(ready)
        for i in grp:
            back(i, i % nsets)
        released[q % 2] = torch.cuda.Event()
        released[q % 2].record(main)
    main.wait_stream(side)


def step_halves(w, sets, inputs, y, first):
    """front(pairs): route and layout of the steps (i, s) in `pairs`, step i
    on buffer set s; back(i, s): dispatch and combine of step i. The fronts
    of a group run as batches of up to MOE_MAX_BATCHES steps, one routing
    launch and one launch per layout pass each (moe_route_batched,
    moe_layout_batched): a group's fronts then cost about one step's
    launches, which shortens the pipeline's fill and leaves fewer launches
    beside the backs. Layout and dispatch are separate launches here even
    where moe_layout_dispatch would fuse them (decode-sized capacity mode):
    the layout is latency-bound, and on the side stream it is hidden."""
    M = _moe()

    def front(pairs):
        ds = [inputs[(first + i) % len(inputs)] for i, _ in pairs]
        for c in range(0, len(pairs), M.MOE_MAX_BATCHES):
            bufs = [sets[s] for _, s in pairs[c:c + M.MOE_MAX_BATCHES]]
            dc = ds[c:c + M.MOE_MAX_BATCHES]
            M.route_batches(bufs, [d["logits"] for d in dc], [d["bias"] for d in dc],
                            w.score_fn, w.groups, w.topk_groups)
            M.layout_batches(bufs)

    def back(i, s):
        d = inputs[(first + i) % len(inputs)]
        sets[s].dispatch(d["x"])
        sets[s].combine(y)

    return front, back


def overlapped_steps(torch, w, sets, inputs, y, first, steps, side, group=PIPE_GROUP,
                     lead=PIPE_LEAD):
    """The steps of serial_steps pipelined on two streams (pipelined()): the
    route and layout of a group of steps run beside the dispatch and combine
    of the group before, on the 2 * group buffer sets in `sets` in turn
    (routing and layout buffers of their own, row buffers shared). Every step
    does all of its work; the results equal those of serial_steps."""
    front, back = step_halves(w, sets, inputs, y, first)
    pipelined(torch, front, back, len(sets), steps, side, group, lead)


GRAPH_WARM_REPLAYS = 3   # untimed replays of a captured graph before the timed one
EVICT_BYTES = 1 << 30    # read before each timed window: more than L2 and the 256 MB MALL
EVICTION = ("a 1 GiB device read before each timed window (evicts L2 and the Infinity Cache "
            "and leaves no dirty lines to write back inside the window)")
_evict_buf = []


def evict_caches(torch):
    """Untimed: read EVICT_BYTES of device memory (a torch reduction, with
    loads that allocate in the caches) and wait, so that the timed window
    that follows starts from HBM, not from cached inputs. A read rather than
    a write: a 1 GiB write left hundreds of MB of dirty lines whose write-back
    then ran inside the window."""
    if not _evict_buf:
        b = torch.empty(EVICT_BYTES // 8, dtype=torch.int64, device="cuda")
        b.fill_(1)
        _evict_buf.append(b)
    torch.amax(_evict_buf[0])
    torch.cuda.synchronize()


def timed_run(torch, run, graph):
    """Wall time of run(): captured into one HIP graph, replayed
    GRAPH_WARM_REPLAYS times untimed (the first uploads it; the first few
    replays of a new graph run 2-5% slower) and once timed; or launched from
    the host once timed (the caller has warmed it up). The caches are evicted
    before the timed window."""
    if graph:
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            run()
        for _ in range(GRAPH_WARM_REPLAYS):
            g.replay()
        torch.cuda.synchronize()
        evict_caches(torch)
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0
    torch.cuda.synchronize()
    evict_caches(torch)
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs the hot path on one GPU only: the simulated destination "
              "ranks are regions of one GPU's HBM and no collective is built, so "
              "--gpus %d is not supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_moe_layout_06_amd as M
    from synth import workloads as W

    if args.calibrate_copy:
        calibrate_copy()
        return

    w = W.WORKLOADS[args.workload]
    # the CPU oracle first: its worker processes start while this process
    # has not touched the GPU yet
    dtype = {"auto": w.dispatch_dtype, "bf16": M.MOE_DTYPE_BF16, "fp8": M.MOE_DTYPE_FP8_E4M3,
             "mxfp8": M.MOE_DTYPE_MXFP8_E4M3}[args.dispatch]
    cpu_base = None
    if args.pass_ == "forward" and not args.no_cpu_baseline:
        cpu_base = cpu_baseline(w, args.seed, dtype)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.pass_ == "backward":
        run_backward(args, w, M, W, torch, np)
        return
    if args.pass_ == "hierarchical":
        run_hierarchical(args, w, M, W, torch, np)
        return
    steps, warm = args.steps, args.warmup

    # ---- inputs, resident in HBM before timing
    n_inputs = steps + warm if w.steps > 1 else 1
    seeds = [w.step_seed0 + i for i in range(n_inputs)] if w.steps > 1 else [args.seed]
    inputs = []
    for s in seeds:
        inp = W.make_inputs(w, s)
        inputs.append(dict(
            logits=torch.from_numpy(inp.logits).to(dev),
            bias=torch.from_numpy(inp.bias).to(dev) if inp.bias is not None else None,
            x=torch.from_numpy(inp.x.view(np.int16)).to(dev)))
    buf = M.LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks,
                                  w.capacity, device=dev, dtype=dtype)

    # layout + dispatch: one launch for decode-sized inputs in capacity mode
    fused = M.moe_layout_dispatch_is_fused(w.tokens, w.top_k, w.capacity)
    # pipelining by default when the steps are replayed from a graph, where
    # the cross-stream order is graph edges; from the host, each step's event
    # record and wait cost more than they hide (decode: 30.4 against 20.4
    # us/step eager, 18.3 against 20.1 replayed)
    if args.overlap is None:
        args.overlap = args.graph
    # pipelined steps: 2 * group sets of routing and layout buffers in
    # turn, the row buffers of `buf` shared (the backs run one after the other)
    group, lead = pipe_shape(w)
    bufs = [buf] + ([buf.sharing_rows() for _ in range(2 * group - 1)]
                    if args.overlap else [])
    side = torch.cuda.Stream() if args.overlap else None

    def front(i):
        d = inputs[i % len(inputs)]
        buf.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups)
        buf.layout_dispatch(d["x"])

    # stand-in expert output (harness): dequantised / scaled rows of step 0
    front(0)
    torch.cuda.synchronize()
    rows = buf.num_rows
    if dtype == M.MOE_DTYPE_FP8_E4M3:
        codes = buf.dispatched[:rows].view(torch.float8_e4m3fn).float()
        sc = buf.scales[:rows].repeat_interleave(128, dim=1)
        y = (codes * sc).to(torch.bfloat16).view(torch.int16).contiguous()
    elif dtype == M.MOE_DTYPE_MXFP8_E4M3:
        codes = buf.dispatched[:rows].view(torch.float8_e4m3fn).float()
        sc = torch.exp2(buf.scales[:rows].float() - 127.0).repeat_interleave(32, dim=1)
        y = (codes * sc).to(torch.bfloat16).view(torch.int16).contiguous()
    elif w.expert_kind == "scaled":
        off = buf.expert_offsets.cpu().numpy()
        e_of_row = torch.from_numpy(np.searchsorted(off[1:], np.arange(rows), side="right")).to(dev)
        c = ((e_of_row + 1).float() / w.experts)[:, None]
        y = (buf.dispatched[:rows].view(torch.bfloat16).float() * c).to(torch.bfloat16)
        y = y.view(torch.int16).contiguous()
    else:
        y = buf.dispatched[:rows].clone()
    rows_live = int((buf.dst_row >= 0).sum().item())
    nbytes = step_bytes(w, rows_live, dtype)
    total_bytes = sum(nbytes.values())

    # ---- warmup
    serial_steps(w, bufs, inputs, y, 0, warm, fuse=not args.graph)
    if args.overlap:
        overlapped_steps(torch, w, bufs, inputs, y, 0, warm, side, group, lead)
    torch.cuda.synchronize()

    # ---- timed steps: back to back, nothing but the path on the stream(s)
    serial_wall = timed_run(torch, lambda: serial_steps(w, bufs, inputs, y, warm, steps,
                                                        fuse=not args.graph), args.graph)
    wall = (timed_run(torch, lambda: overlapped_steps(torch, w, bufs, inputs, y, warm, steps, side,
                                                      group, lead),
                      args.graph) if args.overlap else serial_wall)

    # ---- the same steps again with HIP events between the phases (on the
    # launch stream) for the per-phase times and the roofline; layout and
    # dispatch are one phase when they are one launch
    if fused:
        names = ["route", "layout_dispatch", "combine"]
        calls = [lambda d: buf.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups),
                 lambda d: buf.layout_dispatch(d["x"]), lambda d: buf.combine(y)]
    else:
        names = ["route", "layout", "dispatch", "combine"]
        calls = [lambda d: buf.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups),
                 lambda d: buf.layout(), lambda d: buf.dispatch(d["x"]),
                 lambda d: buf.combine(y)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(steps)]
    for i in range(steps):
        d = inputs[(warm + i) % len(inputs)]
        e = ev[i]
        e[0].record()
        for j, call in enumerate(calls):
            call(d)
            e[j + 1].record()
    torch.cuda.synchronize()

    phase_ms = {n: 0.0 for n in names}
    step_ms = []
    for e in ev:
        for j, n in enumerate(names):
            phase_ms[n] += e[j].elapsed_time(e[j + 1]) / steps
        step_ms.append(e[0].elapsed_time(e[-1]))
    ms_per_step = wall * 1e3 / steps
    value = w.tokens / (ms_per_step * 1e-3)

    # ---- pipelined steps again with wall-clock stamps (latency percentiles)
    stamped = None
    if args.overlap and args.graph:
        front_h, back_h = step_halves(w, bufs, inputs, y, warm)
        stamped = stamped_pipeline(torch, np, front_h, back_h, len(bufs), steps, side, group,
                                   lead)

    # ---- cold steps: 1 GiB write between steps (untimed)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(args.cold_steps):
        flush.zero_()
        d = inputs[i % len(inputs)]
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        buf.route(d["logits"], d["bias"], w.score_fn, w.groups, w.topk_groups)
        buf.layout_dispatch(d["x"])
        buf.combine(y)
        e.record()
        torch.cuda.synchronize()
        cold.append(s.elapsed_time(e))
    del flush

    comb_us = launch_us(torch, lambda: buf.combine(y))
    achieved = nbytes["combine"] / (comb_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "kernel": "combine", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": (load_traffic(nbytes["combine"])
                        or load_kernel_traffic("combine", COMBINE_SOURCES, nbytes["combine"])),
            "algorithmic_bytes_per_launch": nbytes["combine"],
            "launch_us": round(comb_us, 2), "timing": roofline_timing()}

    ceil = ceilings(torch, np)
    out = {
        "metric": "dispatch+combine tokens/s and HBM GB/s (% of peak), DeepSeek-V3 shape, 1 GPU",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "bf16", 1: "fp8e4m3+bf16", 2: "mxfp8e4m3+bf16"}[dtype],
        "data": "synthetic",
        "launch": ("hip graph replay" if args.graph else "eager launches") +
                  ("; steps pipelined on two streams in groups of %d (the first of %d): the "
                   "routes and layouts of one group (batched launches) run beside the "
                   "dispatch and combine of the group before (%d sets of routing and layout "
                   "buffers in turn, row buffers shared)"
                   % (group, min(lead, group), 2 * group)
                   if args.overlap else "; one step after the other on one stream"),
        "serial_ms_per_step": round(serial_wall * 1e3 / steps, 5),
        "cache_eviction": EVICTION,
        "config": {"workload": "%s: T=%d H=%d E=%d k=%d R=%d %s%s, %s dispatch, bf16 combine%s"
                   % (w.name, w.tokens, w.hidden, w.experts, w.top_k, w.ranks,
                      "group-limited sigmoid G=%d kg=%d" % (w.groups, w.topk_groups)
                      if w.groups > 1 else ("sigmoid" if w.score_fn else "softmax"),
                      ", zipf bias" if w.bias == "zipf" else "",
                      {0: "bf16", 1: "fp8 e4m3 (1x128 fp32 scales)",
                       2: "mxfp8 e4m3 (1x32 e8m0 scales)"}[dtype],
                      ", capacity %d" % w.capacity if w.capacity else ""),
                   "tokens": w.tokens, "hidden": w.hidden, "experts": w.experts,
                   "top_k": w.top_k, "ranks": w.ranks, "seed": args.seed},
        "gbps": round(total_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": total_bytes,
        "phases_us": {n: round(v * 1e3, 2) for n, v in phase_ms.items()},
        "phase_bytes": nbytes,
        "event_us_per_step_median": round(float(np.median(step_ms)) * 1e3, 2),
        "event_us_per_step_p99": round(float(np.percentile(step_ms, 99)) * 1e3, 2),
        "pipelined_stamps": stamped,
        "cold_us_per_step": round(float(np.median(cold)) * 1e3, 2) if cold else None,
        "copy_ceiling_gbps": ceil["copy"]["gbps"],
        "ceilings_gbps": ceil,
        "roofline": roof,
        "cpu_baseline": cpu_base,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
