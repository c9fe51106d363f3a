"""The bench line's contract, on the GPU: one JSON line with the throughput,
the roofline object of the dominant kernel and the CPU oracle baseline, for
the smallest workload (64 tokens x 128 channels x 256), run as its own
process the way the bench is run."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_contract():
    cmd = [sys.executable, "bench.py", "--workload", "tiny", "--steps", "3", "--warmup", "2",
           "--preload-ms", "20", "--b2b-ms", "1", "--cpu-seconds", "0.5"]
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "tiny" and d["dtype"] == "int8"
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TOP/s" and rf["peak"] == 5000.0
    # (this workload is a few microseconds of launch-bound work: frac is tiny and
    # rounds to a few units in the fourth decimal)
    assert rf["achieved"] > 0 and 0 <= rf["frac"] < 1
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf              # null: no counters are committed for this workload
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == d["unit"] and isinstance(cpu["sample"], str)
    assert 0 < d["extra"]["rel_frobenius_error_vs_fp32_linear"] < 0.05
    ceiling = d["extra"]["mainloop_ceiling_frac"]
    assert 0 < ceiling["random"] < ceiling["constant"] < 1
