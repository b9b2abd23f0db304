"""bench.py's command-line contract that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_matches_hash_or_is_ignored():
    sys.path.insert(0, ROOT)
    import bench

    t = bench.traffic_for("c3")
    assert t is None or t > 0
    assert bench.traffic_for("no-such-workload") is None


def test_host_record_fields():
    sys.path.insert(0, ROOT)
    import bench

    info = bench.host_info()
    assert info["cpus_available"] >= 1
    assert info["cpu_model"] is None or isinstance(info["cpu_model"], str)
    v = bench.read_sclk_mhz()
    assert v is None or v > 0
