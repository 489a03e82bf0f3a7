"""bench.py end to end on the GPU, on the small workload (T=128, H=256):
one JSON line on stdout with the fields the benchmark contract names, the
roofline entry of the dominant kernel, and consistent timings (needs an
MI355X).  Collected last: it starts bench.py as a child process."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", "1", "--steps", "5", "--warmup", "2",
           "--no-cpu-baseline", "--no-other-workloads", "--no-quant", "--no-groups", "--no-decode", "--no-probe"]
    print("[bench-json] " + " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "cold"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True
    assert d["config"]["workload"] == "tiny" and d["config"]["T"] == 128
    assert d["value"] > 0 and abs(d["value"] * d["ms_per_step"] * 1e-3 - 128) < 1e-6 * 128
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert d["cold"]["scatter_us"] > 0 and d["cold"]["combine_us"] > 0
    print("[bench-json] ok", flush=True)
