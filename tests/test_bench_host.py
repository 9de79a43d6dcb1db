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


def test_inflight_summary_from_counters(tmp_path):
    # LEVEL / active cycles = reads in flight, LEVEL / requests = latency; counters summed over
    # their instances per dispatch, the active cycles taken from the slowest XCD; only the
    # profiled dispatches (after a warm-up step) count
    import sqlite3
    import types

    import bench
    db = sqlite3.connect(str(tmp_path / "run_results.db"))
    db.execute("create table pmc_events (name text, dispatch_id integer, counter_name text, counter_value real)")
    k = "void qkv::sparse_chunk_kernel<128, 4, false, false, 3>"
    rows = []
    n = bench.profiled_dispatches("sparse3")
    for i in range(8 + n):
        warm = i < 8
        for inst in range(2):
            rows.append((k, i, "TCC_EA0_RDREQ_LEVEL_sum", 1.0 if warm else 3.0e6))
            rows.append((k, i, "TCC_EA0_RDREQ_sum", 1.0 if warm else 1.0e3))
        for x in range(8):
            rows.append((k, i, "GRBM_GUI_ACTIVE", 5.0 if warm else (1.0e3 if x == 3 else 10.0)))
    db.executemany("insert into pmc_events values (?, ?, ?, ?)", rows)
    db.commit()
    db.close()
    out = tmp_path / "s.txt"
    bench.summarize_inflight(types.SimpleNamespace(summarize_inflight=("sparse3", str(tmp_path)), out=str(out), cmd="c"))
    row = [l for l in out.read_text().splitlines() if l.startswith(f"| {n} |")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells == [str(n), "2000", "1000", "6000", "3000"]
