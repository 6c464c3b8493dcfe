"""bench.py's host-side rules, checked on the CPU: it measures one GPU and says so for any
other count, and it reports memory traffic only from byte counters that were taken on the
current kernel sources (otherwise null)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=300, env=env)


def test_refuses_more_than_one_gpu():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_refuses_a_multi_rank_launch():
    r = _run([], env=dict(os.environ, WORLD_SIZE="2"))
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_from_counters_on_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    for one in (True, False):
        p = bench.traffic_path("decode", one)
        assert bench.load_traffic("decode", one) is None  # no counters taken
        with open(p, "w") as f:
            json.dump({"kernel_sha": bench.kernel_source_sha(), "hbm_bytes_per_launch": 123.0}, f)
        assert bench.load_traffic("decode", one) == 123.0
        with open(p, "w") as f:
            json.dump({"kernel_sha": "0" * 16, "hbm_bytes_per_launch": 123.0}, f)
        assert bench.load_traffic("decode", one) is None  # taken on other sources
        with open(p, "w") as f:
            f.write("{not json")
        assert bench.load_traffic("decode", one) is None


def test_committed_counter_files_are_complete():
    names = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith("_traffic.json")]
    assert names
    for n in names:
        with open(os.path.join(ROOT, "profiles", n)) as f:
            d = json.load(f)
        assert len(d["kernel_sha"]) == 16 and int(d["kernel_sha"], 16) >= 0
        assert d["hbm_bytes_per_launch"] > 0
        assert d["fetch_kib_per_dispatch"] > 0 and d["write_kib_per_dispatch"] > 0
