"""CPU tests of the measurement helpers in bench.py: the algorithmic byte
counts the roofline divides by, and the source hash that decides whether the
committed HBM-traffic record still describes the combine kernel."""

import json

import pytest

import bench
from synth import workloads as W


def test_dsv3_step_bytes_are_the_documented_figures():
    w = W.WORKLOADS["dsv3"]
    b = bench.step_bytes(w, w.tokens * w.top_k)
    T, H, k = w.tokens, w.hidden, w.top_k
    # combine: every row read once (2H), weights + dst_row (8 per pair), out written
    assert b["combine"] == T * k * 2 * H + T * k * 8 + T * 2 * H == 528744448
    # FP8 dispatch: x read, dst_row read, k copies of H codes + H/128 fp32 scales
    assert b["dispatch"] == T * 2 * H + T * k * 4 + T * k * (H + H // 128 * 4) == 301072384
    assert sum(b.values()) == 834670988


def test_mxfp8_moves_the_same_bytes_as_fp8_at_h_7168():
    # 1x32 byte scales and 1x128 fp32 scales both add H/32 bytes per row
    w = W.WORKLOADS["dsv3"]
    rows = w.tokens * w.top_k
    assert bench.step_bytes(w, rows, 1) == bench.step_bytes(w, rows, 2)


def test_dropped_rows_are_not_counted():
    w = W.WORKLOADS["dsv3"]
    full = bench.step_bytes(w, w.tokens * w.top_k)
    fewer = bench.step_bytes(w, w.tokens * w.top_k - 100)
    assert full["combine"] - fewer["combine"] == 100 * 2 * w.hidden
    assert full["dispatch"] - fewer["dispatch"] == 100 * (w.hidden + w.hidden // 128 * 4)


def test_backward_bytes():
    w = W.WORKLOADS["dsv3"]
    rows = w.tokens * w.top_k
    b = bench.backward_bytes(w, rows)
    T, H, k = w.tokens, w.hidden, w.top_k
    assert b["combine_backward"] == T * H * 2 + 2 * rows * H * 2 + T * k * 12
    assert b["dispatch_backward"] == rows * H * 2 + T * k * 4 + T * H * 2


def test_code_only_drops_comments_and_whitespace():
    src = "int a = 1; // one\n/* block\n comment */ int  b =\n 2;"
    assert bench.code_only(src) == "inta=1;intb=2;"


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_traffic_record_follows_the_code_not_the_comments(tmp_path, monkeypatch):
    src = _write(tmp_path, "k.hip", "// combine\n__global__ void k() { x += 1; }\n")
    monkeypatch.setattr(bench, "COMBINE_SOURCES", [src])
    rec = {"kernel_source_sha256": bench.sha_of([src]), "algorithmic_bytes_per_launch": 1000,
           "traffic_bytes_per_launch": 1234}
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _write(tmp_path, "t.json", json.dumps(rec)))
    assert bench.load_traffic(1000) == 1234
    assert bench.load_traffic(999) is None              # another workload
    # a comment edit keeps the record
    _write(tmp_path, "k.hip", "// the combine kernel\n__global__ void k() {\n  x += 1;\n}\n")
    assert bench.load_traffic(1000) == 1234
    # a code edit drops it
    _write(tmp_path, "k.hip", "__global__ void k() { x += 2; }\n")
    assert bench.load_traffic(1000) is None


def test_missing_traffic_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.load_traffic(1000) is None


def test_committed_traffic_record_describes_the_dsv3_combine():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec["kernel_source_sha256"] != bench.sha_of(bench.COMBINE_SOURCES):
        pytest.skip("the combine code changed since its HBM counters were taken; "
                    "bench.py reports traffic as null until they are taken again")
    w = W.WORKLOADS["dsv3"]
    assert rec["algorithmic_bytes_per_launch"] == bench.step_bytes(w, w.tokens * w.top_k)["combine"]


def test_kernel_traffic_records_follow_kernel_source_and_workload(tmp_path, monkeypatch):
    src = _write(tmp_path, "h.hip", "__global__ void k() { y += 1; }\n")
    recs = [{"kernel": "combine_local", "kernel_source_sha256": bench.sha_of([src]),
             "algorithmic_bytes_per_launch": 500, "traffic_bytes_per_launch": 510},
            {"kernel": "combine_backward", "kernel_source_sha256": bench.sha_of([src]),
             "algorithmic_bytes_per_launch": 900, "traffic_bytes_per_launch": 950}]
    monkeypatch.setattr(bench, "KERNEL_TRAFFIC_FILE", _write(tmp_path, "r.json", json.dumps(recs)))
    assert bench.load_kernel_traffic("combine_local", [src], 500) == 510
    assert bench.load_kernel_traffic("combine_backward", [src], 900) == 950
    assert bench.load_kernel_traffic("combine_local", [src], 900) is None     # other workload
    assert bench.load_kernel_traffic("expand", [src], 500) is None            # no record
    _write(tmp_path, "h.hip", "__global__ void k() { y += 2; }\n")            # code edit
    assert bench.load_kernel_traffic("combine_local", [src], 500) is None
    monkeypatch.setattr(bench, "KERNEL_TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.load_kernel_traffic("combine_backward", [src], 900) is None


def test_committed_kernel_traffic_records_describe_the_dsv3_passes():
    """The records of the hierarchical and backward passes' roofline kernels
    carry the bench's own algorithmic bytes for the DeepSeek-V3 shape, and
    their traffic stays within a few percent of them."""
    with open(bench.KERNEL_TRAFFIC_FILE) as f:
        recs = {d["kernel"]: d for d in json.load(f) if d["workload_key"] == "dsv3"}
    w = W.WORKLOADS["dsv3"]
    rows = w.tokens * w.top_k
    want = {"combine_local": (bench.HIER_SOURCES, None),
            "combine_backward": (bench.COMBINE_SOURCES,
                                 bench.backward_bytes(w, rows)["combine_backward"])}
    for kernel, (sources, alg) in want.items():
        d = recs[kernel]
        if d["kernel_source_sha256"] != bench.sha_of(sources):
            pytest.skip("the %s code changed since its HBM counters were taken" % kernel)
        if alg is not None:
            assert d["algorithmic_bytes_per_launch"] == alg
        assert 1.0 <= d["traffic_bytes_per_launch"] / d["algorithmic_bytes_per_launch"] < 1.08


def test_committed_combine_records_of_other_workloads():
    """The mixtral, qwen3_skew and decode combine records carry the bench's
    own algorithmic combine bytes of their workload, so the forward bench
    line of each finds its record, and their traffic is within a few
    percent."""
    with open(bench.KERNEL_TRAFFIC_FILE) as f:
        recs = {d["workload_key"]: d for d in json.load(f) if d["kernel"] == "combine"}
    assert set(recs) == {"mixtral", "qwen3_skew", "decode"}
    for name, d in recs.items():
        if d["kernel_source_sha256"] != bench.sha_of(bench.COMBINE_SOURCES):
            pytest.skip("the combine code changed since its HBM counters were taken")
        w = W.WORKLOADS[name]
        alg = bench.step_bytes(w, w.tokens * w.top_k)["combine"]
        assert d["algorithmic_bytes_per_launch"] == alg
        assert bench.load_kernel_traffic("combine", bench.COMBINE_SOURCES, alg) \
            == d["traffic_bytes_per_launch"]
        assert 1.0 <= d["traffic_bytes_per_launch"] / alg < 1.02


def test_launch_flags(monkeypatch):
    """Default: graph replay, pipelining decided later (None: it follows the
    launch mode); --eager, --serial and --overlap override."""
    for argv, graph, overlap in ([[], True, None], [["--eager"], False, None],
                                 [["--serial"], True, False], [["--overlap", "--eager"], False, True]):
        monkeypatch.setattr(bench.sys, "argv", ["bench.py"] + argv)
        a = bench.parse()
        assert (a.graph, a.overlap) == (graph, overlap), argv


class _FakeTorch:
    """Just enough of torch.cuda for bench.pipelined: streams are queues of
    operations, events point at the last operation of the stream they were
    recorded on, and a wait makes the next operation of a stream depend on
    it. Every enqueued operation records what it must come after."""

    def __init__(self):
        self.ops = []            # (stream, label, set of op indices it depends on)
        self.current = "main"
        torch_self = self

        class Event:
            def __init__(self):
                self.op = None   # index of the op the event marks, None = nothing

            def record(self, stream):
                self.op = torch_self._last(stream.name)

        class Stream:
            def __init__(self, name="side"):
                self.name = name
                self.pending = set()

            def wait_event(self, e):
                if e.op is not None:
                    torch_self.waits[self.name].add(e.op)

            def wait_stream(self, other):
                last = torch_self._last(other.name)
                if last is not None:
                    torch_self.waits[self.name].add(last)

        class _Ctx:
            def __init__(self, s):
                self.s, self.prev = s, None

            def __enter__(self):
                self.prev, torch_self.current = torch_self.current, self.s.name

            def __exit__(self, *a):
                torch_self.current = self.prev

        self.waits = {"main": set(), "side": set()}
        self.main_stream = Stream("main")
        cuda = type("cuda", (), {})()
        cuda.Event = Event
        cuda.Stream = Stream
        cuda.current_stream = lambda: self.main_stream if self.current == "main" else self.side_stream
        cuda.stream = lambda s: _Ctx(s)
        self.cuda = cuda
        self.side_stream = Stream("side")

    def _last(self, stream):
        for j in range(len(self.ops) - 1, -1, -1):
            if self.ops[j][0] == stream:
                return j
        return None

    def op(self, label):
        s = self.current
        deps = set(self.waits[s])
        prev = self._last(s)
        if prev is not None:
            deps.add(prev)
        self.waits[s] = set()
        self.ops.append((s, label, deps))

    def before(self, a, b):
        """Op a happens before op b (transitively)."""
        todo, seen = [b], set()
        while todo:
            x = todo.pop()
            for d in self.ops[x][2]:
                if d == a:
                    return True
                if d not in seen:
                    seen.add(d)
                    todo.append(d)
        return False


def test_pipeline_groups():
    assert [list(g) for g in bench.pipeline_groups(10, 4, 1)] == [[0], [1, 2, 3, 4],
                                                                  [5, 6, 7, 8], [9]]
    assert [list(g) for g in bench.pipeline_groups(9, 4, 4)] == [[0, 1, 2, 3], [4, 5, 6, 7],
                                                                 [8]]
    assert [list(g) for g in bench.pipeline_groups(1, 4, 1)] == [[0]]
    assert bench.pipeline_groups(0, 4, 1) == []
    for steps in range(0, 30):
        for group in (1, 2, 4, 8):
            for lead in (1, 2, 3, 4, 9):
                gs = bench.pipeline_groups(steps, group, lead)
                assert [i for g in gs for i in g] == list(range(steps))
                assert all(1 <= len(g) <= group for g in gs)


@pytest.mark.parametrize("group,steps,lead", [(4, 13, 4), (1, 5, 1), (2, 8, 2), (4, 13, 1),
                                              (4, 20, 4), (4, 3, 4), (2, 9, 1), (4, 14, 3)])
def test_pipelined_step_dependencies(group, steps, lead):
    """bench.pipelined on a fake torch: the side stream runs the fronts, the
    current stream the backs, each in step order; every back comes after its
    own front, every front after the work queued before the call and after
    the back of the step that last used its buffer set; the fronts of a group
    do not wait for the backs of the group before (they run beside them)."""
    ft = _FakeTorch()
    ft.op(("before",))
    nsets = 2 * group
    bench.pipelined(ft, lambda pairs: [ft.op(("front", i, s)) for i, s in pairs],
                    lambda i, s: ft.op(("back", i, s)), nsets, steps, ft.side_stream, group, lead)
    idx = {op[1]: n for n, op in enumerate(ft.ops)}
    before = idx[("before",)]
    for i in range(steps):
        s = i % nsets
        f, b = idx[("front", i, s)], idx[("back", i, s)]
        assert ft.ops[f][0] == "side" and ft.ops[b][0] == "main"
        assert ft.before(f, b), i
        assert ft.before(before, f), i
        if i >= nsets:                        # the previous user of set s is done first
            assert ft.before(idx[("back", i - nsets, s)], f), i
    groups = bench.pipeline_groups(steps, group, lead)
    for q in range(1, len(groups)):
        for i in groups[q]:
            for j in groups[q - 1]:
                assert not ft.before(idx[("back", j, j % nsets)],
                                     idx[("front", i, i % nsets)]), (i, j)
