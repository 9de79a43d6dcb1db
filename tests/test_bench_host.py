"""Host-side behaviour of bench.py: the one-GPU guard, and the rule that the counter-based
traffic figure is used only for the kernel source it was measured on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def _summary(path, source_hash, hbm):
    with open(path, "w") as f:
        f.write("# summary\n| kernel | a | b |\n")
        f.write(f"hbm_bytes_per_launch: {hbm}\nkernel_source_hash: {source_hash}\n")


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    p = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.read_traffic() is None                       # no summary
    _summary(p, bench._dense_source_hash(), 171000000)
    assert bench.read_traffic() == 171000000                  # taken on this source
    _summary(p, "0" * 16, 171000000)
    assert bench.read_traffic() is None                       # taken on another source
