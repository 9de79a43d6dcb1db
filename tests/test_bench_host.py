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
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    for key, (fname, _, srcs) in bench.TRAFFIC.items():
        p = tmp_path / "profiles" / fname
        assert bench.read_traffic(key) is None                  # no summary
        _summary(p, bench.source_hash(srcs), 171000000)
        assert bench.read_traffic(key) == 171000000             # taken on this source
        _summary(p, "0" * 16, 171000000)
        assert bench.read_traffic(key) is None                  # taken on another source


def test_cpu_info_names_the_host():
    model, nproc = bench.cpu_info()
    assert nproc >= 1 and isinstance(model, str)


def test_counter_mean_takes_the_profiled_dispatches(tmp_path):
    # a warm-up step's dispatches of the same kernel (another loop's instance) come first and
    # must not enter the per-launch mean
    import sqlite3

    import bench
    db = sqlite3.connect(str(tmp_path / "run_results.db"))
    db.execute("create table pmc_events (name text, dispatch_id integer, counter_name text, counter_value real)")
    rows = [("void qkv::dense_split_kernel<128, 2, 4, false, false>", i, "FETCH_SIZE", 900.0) for i in range(8)]
    rows += [("void qkv::dense_split_kernel<128, 1, 4, false, false>", 8 + i, "FETCH_SIZE", 500.0) for i in range(24)]
    rows += [("void qkv::dense_split_kernel<128, 1, 4, false, false>", 40 + i, "WRITE_SIZE", 7.0) for i in range(24)]
    db.executemany("insert into pmc_events values (?, ?, ?, ?)", rows)
    db.commit()
    db.close()
    assert bench._counter_per_dispatch(str(tmp_path), "FETCH_SIZE", ("dense_split_kernel",))["dense_split_kernel"] == \
        ((8 * 900.0 + 24 * 500.0) / 32, 32)
    assert bench._counter_per_dispatch(str(tmp_path), "FETCH_SIZE", ("dense_split_kernel",),
                                       bench.profiled_dispatches("dense1"))["dense_split_kernel"] == (500.0, 24)
    assert bench.profiled_dispatches("select") == 3
