"""bench.py's JSON line: one short run on the decode S=1 workload (the
smallest configuration) as a child process, checked field by field against
the line's documented contract (metric and throughput, the dominant
kernel's roofline object, the oracle's CPU baseline, the workload's name)."""
import json
import math
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    print("[bench] decode1, 3 steps", flush=True)
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "decode1",
           "--steps", "3", "--warmup", "1", "--no-train", "--no-workloads",
           "--decode-steps", "40"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and math.isfinite(d["value"]) and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None or d["vs_baseline"] > 0
    assert d["config"]["workload"] == "decode1"
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["achieved"] > 0 and rf["peak"] > 0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == d["unit"] and isinstance(cb["sample"], str) and cb["sample"]
    assert d["status"] == 0
