"""bench.py's host-side logic, without a GPU: the algorithmic byte counts it
prices the roofline with, the refusal of more than one GPU, and the rule
that a stored PMC traffic figure is reported only for the kernel source it
was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_bytes_of_the_stress_workload():
    # 4096 rows x 200064 bf16 columns, 8 shards of 25008, 8192-column blocks:
    # M = 4 slots per shard; per row V*2 logits bytes + S*M*8 statistics
    # written and read back + 8 bytes of id and value.
    assert bench.slots(25008, 8, 8192) == 4
    assert bench.slots(25008, 8, 1024) == 26
    alg = bench.algorithmic_bytes()
    assert alg["top_tokens"] == 4096 * (200064 * 2 + 8 * 4 * 8 * 2 + 8) == 1_641_054_208
    # verification statistics: 682 x 5 draft rows (8192-blocks) and 682
    # bonus rows (1024-blocks), logits plus statistics written
    assert alg["verify_stats"] == (682 * 5 * (200064 * 2 + 8 * 4 * 8)
                                   + 682 * (200064 * 2 + 8 * 26 * 8)) == 1_639_331_584
    assert alg["greedy_verify"] > 0


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    rec = {"hbm_bytes_per_launch": 123, "kernel_source_hash": bench.kernel_source_hash()}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic() == 123
    rec["kernel_source_hash"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None
