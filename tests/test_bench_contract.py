"""bench.py's measurement contract on the CPU: the multi-GPU refusal, the algorithmic work it
divides by (against hand-computed figures for the T=8192 workload), and the rule that the
traffic figure is reported only while the kernel sources match the committed counters."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from quantized_expert_grouped_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_work_t8k():
    """T = 8192, H = 2048, F = 512, E = 512, K = 10, Q4_1, every expert active."""
    c = synth.Case.__new__(synth.Case)
    c.T, c.H, c.F, c.E, c.K, c.wtype = 8192, 2048, 512, 512, 10, synth.Q4_1
    c.expert_bytes = synth.expert_bytes(2048, 512, synth.Q4_1)
    w = bench.algorithmic_work(c, 512)
    R = 81920
    assert c.expert_bytes == 1966080                    # 3 * 2048 * 512 / 32 blocks * 20 B
    assert w["gate_up"] == ("ops", 343597383680)        # 4 R F H
    assert w["down"] == ("ops", 171798691840)           # 2 R H F
    assert w["gather"] == ("bytes", 2 * 512 * 1966080)  # read + write of every active expert
    # quantize: x read once (4 T H), slots (4 R), q8_1 rows written (R * H/128 * 144)
    assert w["quantize"] == ("bytes", 4 * 8192 * 2048 + 4 * R + R * 16 * 144)
    # combine: Dm rows read (4 R H), slot and weight (8 R), out written (4 T H)
    assert w["combine"] == ("bytes", 4 * R * 2048 + 8 * R + 4 * 8192 * 2048)
    assert w["route"] == ("bytes", 4 * 8192 * 512 + 8 * R)


def test_traffic_figure_follows_the_source_hash(tmp_path, monkeypatch):
    """A stage's traffic is read from profiles/traffic_<workload>.txt only while the hash of that
    stage's kernel sources matches the one recorded beside it."""
    p = tmp_path / "traffic_t8k.txt"
    p.write_text("# header\n"
                 f"traffic gate_up 929143756 {bench.stage_source_hash('gate_up')}\n"
                 f"traffic combine 738000000 {'0' * 16}\n")
    monkeypatch.setattr(bench, "traffic_path", lambda w: str(p) if w == "t8k" else "/nonexistent")
    assert bench.measured_traffic("gate_up", "t8k") == 929143756
    assert bench.measured_traffic("combine", "t8k") is None        # stale hash
    assert bench.measured_traffic("quantize", "t8k") is None       # no line
    assert bench.measured_traffic("gate_up", "t2k") is None        # no file
    monkeypatch.setattr(bench, "stage_source_hash", lambda st: "1" * 16)
    assert bench.measured_traffic("gate_up", "t8k") is None


def test_committed_traffic_summaries_parse():
    """Every committed summary's traffic lines name a known stage, a byte count and a hash."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.txt")):
        lines = [l.split() for l in open(path) if l.startswith("traffic ")]
        assert lines, path
        for f in lines:
            assert len(f) == 4 and f[1] in bench.STAGE_SOURCES and int(f[2]) > 0 and len(f[3]) == 16
