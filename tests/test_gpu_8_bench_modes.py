"""bench.py's modes on the GPU, each in a child process on the tiny workload: the JSON line it
prints carries the fields the benchmark contract names, and a positive rate."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MODES = [
    ("default", []),
    ("streamed", ["--walk", "streamed", "--ring-slots", "4"]),
    ("packed", ["--walk", "packed"]),
    ("graph", ["--graph"]),
    ("cold", ["--cold-mib", "64"]),
    ("d4", ["--act-d4"]),
    ("quant_ab", ["--quant-ab"]),
]


@pytest.mark.parametrize("mode", MODES, ids=[m[0] for m in MODES])
def test_bench_mode_prints_one_contract_line(mode):
    name, extra = mode
    note(f"bench mode {name}")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
           "--warmup", "1", "--no-cpu-baseline", *extra]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    b = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["value"] > 0 and b["ms_per_step"] > 0
    if name == "quant_ab":        # its own sizes: the quantiser page's 2K / 8K / 32K tokens
        assert [r["T"] for r in b["results"]] == [2048, 8192, 32768]
        assert all(r["cold_scatter_ms"] > 0 and r["warm_gather_ms"] > 0 for r in b["results"])
        return
    assert b["config"]["workload"].startswith("tiny")
    if name == "default":  # (the tiny case's fractions round to zero)
        rf = b["roofline"]
        for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
            assert key in rf, key
        assert rf["unit"] in ("TOP/s", "GB/s") and rf["peak"] > 0 and rf["frac"] >= 0
    if name == "cold":
        assert "cold" in b["metric"] and "cache" in b["config"]
