"""bench.py end to end on the tiny layer: one JSON line with the fields its
readers rely on, in both launch modes. The run is a child process, as the
driver runs it."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
          "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "launch",
          "serial_ms_per_step", "roofline", "cpu_baseline", "phases_us", "cache_eviction")


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "8", "--warmup", "2", "--cold-steps", "1",
                        "--cpu-seconds", "0.5", *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("args,pipelined", [((), True), (("--serial", "--eager"), False)])
def test_bench_line(args, pipelined):
    d = _run(*args)
    for f in FIELDS:
        assert f in d, f
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["serial_ms_per_step"] > 0
    assert abs(d["value"] * d["ms_per_step"] * 1e-3 - d["config"]["tokens"]) < 1e-3 * d["config"]["tokens"]
    assert ("pipelined" in d["launch"]) == pipelined
    if not pipelined:
        assert d["ms_per_step"] == d["serial_ms_per_step"]
        assert d["pipelined_stamps"] is None
    else:
        st = d["pipelined_stamps"]
        assert 0 < st["interval_us_p50"] <= st["interval_us_p99"]
        assert 0 < st["latency_us_p50"] <= st["latency_us_p99"]
        assert st["latency_us_p50"] >= st["interval_us_p50"] * 0.5
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert 0 < roof["frac"] <= 1.0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert 1 <= cpu["cores"] <= cpu["host_cores"] and cpu["all_cores"]["workers"] == cpu["cores"]
    for leg in ("all_cores", "single_thread"):
        assert set(cpu[leg]["phases_s"]) == {"route", "layout_dispatch", "combine"}
        assert cpu[leg]["value"] > 0
